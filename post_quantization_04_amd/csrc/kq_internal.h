// Internal declarations shared by the kernel modules of libkq (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "kq.h"

namespace kq {

// Records a message for kq_last_error() and returns `s`.
kq_status fail(kq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Turns a launch error into KQ_EDEVICE with the kernel's name.
kq_status check_launch(const char* what);

// Brackets one kernel launch with HIP events when kernel timing is enabled
// for this kernel name (kq_timing_enable); otherwise does nothing.
class LaunchTimer {
 public:
  LaunchTimer(const char* name, hipStream_t st);
  ~LaunchTimer();
  LaunchTimer(const LaunchTimer&) = delete;
  LaunchTimer& operator=(const LaunchTimer&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  hipEvent_t begin_ = nullptr;
};

// Number of XCDs on MI355X; workgroups are dispatched to them round robin.
constexpr int kXcds = 8;
// Compute units on MI355X (32 per XCD).
constexpr int kCus = 256;

// ---------------------------------------------------------------------------
// module launchers (arguments already validated by the API layer)
// ---------------------------------------------------------------------------

// covariance (syrk.hip)
size_t syrk_workspace(int64_t rows, int64_t d);
kq_status syrk_run(const uint16_t* a, int64_t rows, int64_t d, int64_t lda, float alpha, float beta,
                   float* h, void* ws, hipStream_t st);
size_t xcov_workspace(int64_t rows, int64_t d);
kq_status xcov_run(const uint16_t* a, const uint16_t* b, int64_t rows, int64_t d, int64_t lda, int64_t ldb,
                   float alpha, float beta, const float* c_in, float* c, void* ws, hipStream_t st);

// GPTAQ drift correction (gptaq.hip)
size_t gptaq_workspace(int64_t dout, int64_t din);
kq_status gptaq_target_run(double* w, const float* d2, const float* r, int64_t dout, int64_t din, int32_t* info,
                           void* ws, hipStream_t st);

// trace score (score.hip)
kq_status score_run(const float* h_x, int64_t din, const float* h_g, int64_t dout, int mode,
                    double* score, hipStream_t st);

// BiIP (biip.hip)
size_t biip_workspace(int64_t dout, int64_t din);
kq_status biip_run(const void* w, int w_dtype, int64_t dout, int64_t din, double* w_out, float* h_x,
                   float* h_g, const kq_rot* rot_in, const kq_rot* rot_out, uint32_t flags,
                   double* s_x, double* s_g, void* ws, hipStream_t st);
kq_status biip_transform_run(float* m, int64_t n, const kq_rot* rot, const double* s, void* ws, hipStream_t st);

// damped Cholesky factor of the inverse (chol.hip)
size_t chol_workspace(int64_t d);
kq_status chol_run(float* h, int64_t d, float damp, int32_t* info, void* ws, hipStream_t st);

// OBS sweep (obs.hip)
size_t obs_workspace(int64_t dout, int64_t din, int block);
kq_status obs_run(double* w, const float* r, int64_t dout, int64_t din, int bits, int group, int block,
                  uint8_t* codes, float* scales, uint8_t* zeros, double* preround, void* ws,
                  hipStream_t st);

// Kronecker layer loss (loss.hip)
size_t loss_workspace(int64_t dout, int64_t din);
kq_status loss_run(const double* w_hat, const void* w, int w_dtype, int64_t dout, int64_t din, const float* h_x,
                   const float* h_g, double* loss, void* ws, hipStream_t st);

// packed codes and the decode matvec (decode.hip)
int container_bits(int bits);
int decode_cpl(int64_t din, int64_t tokens);
size_t decode_workspace(int64_t dout, int64_t din, int64_t tokens);
size_t decode_lds_bytes(int64_t dout, int64_t din, int64_t tokens, bool in_side, bool out_rot);
kq_status pack_run(const uint8_t* codes, int64_t rows, int64_t cols, int bits, uint32_t* packed, hipStream_t st);
kq_status decode_run(const kq_decode_layer* layers, int n_layers, int64_t din, int bits, int group,
                     const double* s_x, const kq_rot* rot_in, const float* x, int64_t tokens, void* ws,
                     hipStream_t st);
// Device address of the decode module's fixed scratch array on the current device (looked up
// once per device and kept); KQ_EDEVICE if the runtime cannot resolve it.
kq_status decode_static_scratch(void** ptr);

}  // namespace kq
