// Host-side check of the C-ABI layer under AddressSanitizer: every entry point
// of include/kda.h is called with arguments that its validation rejects, or
// that make it a no-op, or that pass validation and then fail at the first
// HIP call on a host without a GPU.  Fake, aligned device addresses stand in
// for the buffers (validation compares addresses and sizes and never
// dereferences them).  Built with the library's host code instrumented
// (-Xarch_host -fsanitize=address); exits 1 on a wrong status, and
// AddressSanitizer aborts on any invalid host memory access.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda.h"

namespace {

int failures = 0;

void expect(kda_status_t got, kda_status_t want, const char* what, int line) {
    if (got != want) {
        std::fprintf(stderr, "line %d: %s returned %d (%s), expected %d\n", line, what, (int)got,
                     kda_status_string(got), (int)want);
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

constexpr uintptr_t kA = uintptr_t(1) << 20;  // fake buffers 1 MiB apart
template <typename T>
T* at(uintptr_t addr) {
    return reinterpret_cast<T*>(addr);
}
template <typename T>
T* buf(int i) {
    return at<T>(kA * uintptr_t(i + 1));
}

const uint16_t* cq() { return buf<const uint16_t>(0); }
const uint16_t* ck() { return buf<const uint16_t>(1); }
const uint16_t* cv() { return buf<const uint16_t>(2); }
const float* cg() { return buf<const float>(3); }
const float* cb() { return buf<const float>(4); }

void chunk_forward() {
    const float inf = INFINITY, nan = NAN;
    uint16_t* out = buf<uint16_t>(5);
    EXPECT(kda_chunk_fwd(cq(), ck(), cv(), cg(), cb(), 1.f, nullptr, out, nullptr, -1, 4, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd(cq(), ck(), cv(), cg(), cb(), inf, nullptr, out, nullptr, 1, 4, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd(cq(), ck(), cv(), cg(), cb(), nan, nullptr, out, nullptr, 1, 4, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd(nullptr, ck(), cv(), cg(), cb(), 1.f, nullptr, out, nullptr, 1, 4, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd(at<const uint16_t>(kA + 8), ck(), cv(), cg(), cb(), 1.f, nullptr, out,
                         nullptr, 1, 4, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd(cq(), ck(), cv(), cg(), cb(), 1.f, nullptr, at<uint16_t>(kA + 256), nullptr,
                         1, 4, 1, nullptr),
           KDA_ERR_INVALID_ARG);  // out over q
    EXPECT(kda_chunk_fwd(cq(), ck(), cv(), cg(), cb(), 1.f, nullptr, out, nullptr, 0, 4, 1, nullptr),
           KDA_OK);
    EXPECT(kda_chunk_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 1.f, nullptr, nullptr, nullptr, 1,
                         0, 1, nullptr),
           KDA_OK);
    float* hs = buf<float>(7);
    EXPECT(kda_chunk_fwd(cq(), ck(), cv(), cg(), cb(), 1.f, hs, out, hs, 1, 0, 1, nullptr), KDA_OK);

    EXPECT(kda_chunk_fwd_f32(buf<const float>(0), buf<const float>(1), buf<const float>(2), cg(),
                             cb(), 1.f, nullptr, buf<float>(5), nullptr, 1, -1, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd_f32(buf<const float>(0), buf<const float>(1), buf<const float>(2), cg(),
                             cb(), 1.f, hs, buf<float>(5), at<float>(kA * 8 + 4096), 1, 4, 1,
                             nullptr),
           KDA_ERR_INVALID_ARG);  // h0 and hT partly overlapping
    EXPECT(kda_chunk_fwd_g16(cq(), ck(), cv(), buf<const uint16_t>(3), cb(), 1.f, nullptr, out,
                             nullptr, 1, 4, -3, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd_g16(cq(), ck(), cv(), buf<const uint16_t>(3), cb(), 1.f, nullptr, out,
                             nullptr, 1, 4, 0, nullptr),
           KDA_OK);
    // the entry point without allocation: validation, then its size limit
    EXPECT(kda_chunk_fwd_noalloc(cq(), ck(), cv(), cg(), cb(), nan, nullptr, out, nullptr, 1, 4, 1,
                                 nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd_noalloc(cq(), ck(), cv(), cg(), cb(), 1.f, nullptr, out, nullptr, 0, 4, 1,
                                 nullptr),
           KDA_OK);
    auto far = [](int i) { return uintptr_t(i + 1) << 36; };
    EXPECT(kda_chunk_fwd_noalloc(at<const uint16_t>(far(0)), at<const uint16_t>(far(1)),
                                 at<const uint16_t>(far(2)), at<const float>(far(3)),
                                 at<const float>(far(4)), 1.f, nullptr, at<uint16_t>(far(5)),
                                 nullptr, 1, 640, 1024, nullptr),
           KDA_ERR_UNSUPPORTED);
}

void chunk_conv() {
    const float* w = buf<const float>(8);
    uint16_t* out = buf<uint16_t>(5);
    EXPECT(kda_chunk_fwd_conv(cq(), ck(), cv(), w, buf<const float>(9), buf<const float>(10), nullptr,
                              nullptr, cg(), cb(), 1.f, nullptr, nullptr, out, nullptr, -1, 4, 1,
                              nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_chunk_fwd_conv(cq(), ck(), cv(), nullptr, buf<const float>(9), buf<const float>(10),
                              nullptr, nullptr, cg(), cb(), 1.f, nullptr, nullptr, out, nullptr, 1, 4,
                              1, nullptr),
           KDA_ERR_INVALID_ARG);
    uint16_t* cs = buf<uint16_t>(11);
    EXPECT(kda_chunk_fwd_conv(cq(), ck(), cv(), w, buf<const float>(9), buf<const float>(10), cs,
                              at<uint16_t>(kA * 12 + 512), cg(), cb(), 1.f, nullptr, nullptr, out,
                              nullptr, 1, 4, 1, nullptr),
           KDA_ERR_INVALID_ARG);  // conv state in and out partly overlapping
    EXPECT(kda_chunk_fwd_conv(cq(), ck(), cv(), w, buf<const float>(9), buf<const float>(10), nullptr,
                              nullptr, cg(), cb(), 1.f, nullptr, nullptr, out, nullptr, 1, 4, 0,
                              nullptr),
           KDA_OK);
}

void steps() {
    float* S = buf<float>(6);
    uint16_t* out = buf<uint16_t>(5);
    EXPECT(kda_recurrent_step(cq(), ck(), cv(), cg(), cb(), 1.f, S, out, -1, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_recurrent_step(cq(), ck(), cv(), cg(), cb(), 1.f, nullptr, out, 1, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_recurrent_step(cq(), ck(), cv(), cg(), cb(), 1.f, S, at<uint16_t>(kA * 7 + 64), 1, 1,
                              nullptr),
           KDA_ERR_INVALID_ARG);  // out over the state
    EXPECT(kda_recurrent_step(cq(), ck(), cv(), cg(), cb(), 1.f, S, out, 0, 1, nullptr), KDA_OK);
    EXPECT(kda_recurrent_step_f32(buf<const float>(0), buf<const float>(1), buf<const float>(2), cg(),
                                  cb(), -INFINITY, S, buf<float>(5), 1, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_recurrent_step_f32(buf<const float>(0), buf<const float>(1), buf<const float>(2), cg(),
                                  cb(), 1.f, S, buf<float>(5), 1, 0, nullptr),
           KDA_OK);
    const float* w = buf<const float>(8);
    uint16_t* cs = buf<uint16_t>(11);
    EXPECT(kda_recurrent_step_conv(cq(), ck(), cv(), w, buf<const float>(9), buf<const float>(10),
                                   at<uint16_t>(kA * 1 + 128), cg(), cb(), 1.f, S, nullptr, out, 1,
                                   1, nullptr),
           KDA_ERR_INVALID_ARG);  // conv state over an input
    EXPECT(kda_recurrent_step_conv(cq(), ck(), cv(), w, buf<const float>(9), buf<const float>(10), cs,
                                   cg(), cb(), 1.f, S, nullptr, out, 0, 1, nullptr),
           KDA_OK);
}

void step_backward() {
    const float* f = buf<const float>(0);
    float* dbeta = buf<float>(12);
    EXPECT(kda_recurrent_step_bwd_f32(f, buf<const float>(1), buf<const float>(2), cg(), cb(), 1.f,
                                      buf<const float>(5), buf<const float>(6), buf<float>(7),
                                      buf<float>(8), buf<float>(9), buf<float>(10), buf<float>(11),
                                      dbeta, -1, 1, nullptr),
           KDA_ERR_INVALID_ARG);
    EXPECT(kda_recurrent_step_bwd_f32(f, buf<const float>(1), buf<const float>(2), cg(), cb(), 1.f,
                                      buf<const float>(5), buf<const float>(6), buf<float>(7),
                                      at<float>(kA * 1 + 128), buf<float>(9), buf<float>(10),
                                      buf<float>(11), dbeta, 1, 1, nullptr),
           KDA_ERR_INVALID_ARG);  // dq over q
    EXPECT(kda_recurrent_step_bwd(cq(), ck(), cv(), cg(), cb(), 1.f, buf<const float>(5),
                                  buf<const uint16_t>(6), buf<float>(7), buf<uint16_t>(8),
                                  buf<uint16_t>(9), buf<uint16_t>(10), buf<float>(11), dbeta, 1, 0,
                                  nullptr),
           KDA_OK);
}

void chunk_backward() {
    auto bwd = [](int B, int T, int H, float scale, uintptr_t spacing, int dup_to = -1,
                  int dup_from = -1) {
        uintptr_t a[14];
        for (int i = 0; i < 14; ++i) a[i] = spacing * uintptr_t(i + 1);
        if (dup_to >= 0) a[dup_to] = a[dup_from];
        return kda_chunk_bwd_f32(at<const float>(a[0]), at<const float>(a[1]), at<const float>(a[2]),
                                 at<const float>(a[3]), at<const float>(a[4]), scale,
                                 at<const float>(a[5]), at<const float>(a[6]), at<const float>(a[7]),
                                 at<float>(a[8]), at<float>(a[9]), at<float>(a[10]), at<float>(a[11]),
                                 at<float>(a[12]), at<float>(a[13]), B, T, H, nullptr);
    };
    EXPECT(bwd(-1, 4, 1, 1.f, kA), KDA_ERR_INVALID_ARG);
    EXPECT(bwd(1, 4, 1, NAN, kA), KDA_ERR_INVALID_ARG);
    EXPECT(bwd(1, 4, 1, 1.f, kA, 8, 9), KDA_ERR_INVALID_ARG);    // dq at dk
    EXPECT(bwd(1, 4, 1, 1.f, kA, 13, 7), KDA_ERR_INVALID_ARG);   // dh0 at dhT
    EXPECT(bwd(0, 4, 1, 1.f, kA), KDA_OK);
    // split into segments and passed to the device: the first HIP call fails here
    EXPECT(bwd(1, 64 * 2048 + 1, 4096, 1.f, uintptr_t(1) << 40), KDA_ERR_HIP);
    EXPECT(bwd(2, 64, (1 << 21) + 1, 1.f, uintptr_t(1) << 46), KDA_ERR_UNSUPPORTED);
    EXPECT(kda_chunk_bwd(cq(), ck(), cv(), cg(), cb(), 1.f, nullptr, buf<const uint16_t>(6), nullptr,
                         buf<uint16_t>(8), buf<uint16_t>(9), buf<uint16_t>(10), buf<float>(11),
                         buf<float>(12), nullptr, 1, 4, -1, nullptr),
           KDA_ERR_INVALID_ARG);
}

void status_strings() {
    const char* names[] = {"KDA_OK", "KDA_ERR_INVALID_ARG", "KDA_ERR_UNSUPPORTED", "KDA_ERR_HIP",
                           "KDA_ERR_NO_MEMORY", "KDA_ERR_PRECONDITION", "KDA_ERR_DEVICE"};
    for (int c = 0; c < 7; ++c) {
        const char* s = kda_status_string((kda_status_t)c);
        if (!s || std::strncmp(s, names[c], std::strlen(names[c])) != 0) {
            std::fprintf(stderr, "status %d: %s\n", c, s ? s : "(null)");
            ++failures;
        }
    }
    const char* u = kda_status_string((kda_status_t)99);
    if (!u || !std::strstr(u, "unknown")) ++failures;
    EXPECT(kda_trim_workspace(), KDA_OK);
}

}  // namespace

int main() {
    // The fake addresses must never reach a kernel: on a host with a GPU a
    // call that passes validation would launch on them, so stop there.
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
        std::printf("skipped: a GPU is visible\n");
        return 77;
    }
    chunk_forward();
    chunk_conv();
    steps();
    step_backward();
    chunk_backward();
    status_strings();
    if (failures) {
        std::fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    std::printf("kda ABI checks passed under AddressSanitizer\n");
    return 0;
}
