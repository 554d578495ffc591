// Opt-in checks of the KDA_DEBUG_CHECKS mode (internal; the mode is read from
// the environment on every call, so a caller can switch it on and off).
//
// With the mode on, an entry point first scans its inputs on the device for
// the documented preconditions: the log-decay g within [-5, 0] (the bound the
// pages give for the decay gate: 深入 Kimi-K3 thread, KDA paragraph; Kimi K3
// 架构全景 page, section 02) and every value finite.  It synchronises its
// stream, reads the result back and returns KDA_ERR_PRECONDITION before
// launching anything else.  After the work it synchronises again and returns
// KDA_ERR_DEVICE if a kernel's bounded wait gave up (the outputs are then
// invalid).  The status words are a small device array per GPU written only
// with vector stores.  The mode synchronises, so it is not for graph capture.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// Spin limit of the bounded LDS waits: about a second of polling, never
// reached when the waves of a workgroup run (they are resident together).
constexpr unsigned kDefaultSpinLimit = 1u << 23;

// Scans n values at p (fp32, or bf16 bit patterns when bf16) on `stream`:
// flags[0] = 1 if lo <= hi and a value lies outside [lo, hi] (NaN included),
// flags[1] = 1 if a value is not finite.
hipError_t launch_check(const void* p, size_t n, bool bf16, float lo, float hi,
                        unsigned* flags, hipStream_t stream);

class DebugScope {
public:
    explicit DebugScope(hipStream_t stream);
    bool on() const { return on_; }
    // KDA_OK, or KDA_ERR_HIP if the mode is on and its set-up failed
    kda_status_t setup_status() const { return setup_; }
    // the value checks; no-ops when the mode is off or p is NULL
    void finite(const float* p, size_t n) { check(p, n, false, 1.f, 0.f); }
    void finite(const uint16_t* p, size_t n) { check(p, n, true, 1.f, 0.f); }
    void decay(const float* p, size_t n) { check(p, n, false, -5.f, 0.f); }
    void decay(const uint16_t* p, size_t n) { check(p, n, true, -5.f, 0.f); }
    // after the checks: KDA_ERR_PRECONDITION, KDA_ERR_HIP or KDA_OK (always
    // KDA_OK when the mode is off)
    kda_status_t inputs_status();
    // where a bounded wait records giving up (NULL when the mode is off), and
    // the spin limit to use (KDA_DEBUG_SPIN_LIMIT in the mode, to force the
    // path from the host; the default otherwise)
    unsigned* abort_word() const { return on_ ? flags_ + 2 : nullptr; }
    unsigned spin_limit() const { return spin_; }
    // after the work: KDA_ERR_DEVICE, KDA_ERR_HIP or KDA_OK
    kda_status_t device_status();

private:
    void check(const void* p, size_t n, bool bf16, float lo, float hi);
    hipStream_t stream_;
    bool on_ = false;
    kda_status_t setup_ = KDA_OK;
    unsigned* flags_ = nullptr;
    unsigned spin_ = kDefaultSpinLimit;
    bool launch_failed_ = false;
};

}  // namespace kda
