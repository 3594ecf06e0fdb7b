// C ABI of libkq: argument validation, error reporting and dispatch.
//
// Every check here runs on the host before anything is enqueued, so invalid
// calls fail the same way with or without a GPU present.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>
#include <algorithm>

#include "kq_internal.h"

namespace kq {

namespace {
thread_local char g_error[512] = "";
}

kq_status fail(kq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return s;
}

kq_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return KQ_OK;
}

}  // namespace kq

using kq::fail;

namespace {

constexpr int64_t kMaxDim = 65536;

bool rot_ok(const kq_rot* r, int64_t n, const char* side) {
  if (!r) {
    fail(KQ_EINVAL, "%s rotation spec is NULL", side);
    return false;
  }
  if (r->n != n) {
    fail(KQ_EINVAL, "%s rotation has n = %lld, expected %lld", side, (long long)r->n, (long long)n);
    return false;
  }
  if (r->m < 1 || r->m > KQ_MAX_ODD || (r->m % 2) == 0 || r->log2p < 0 || r->log2p > 15 ||
      (int64_t(r->m) << r->log2p) != n) {
    fail(KQ_EINVAL, "%s rotation: n = %lld is not m * 2^log2p with odd m <= %d (m = %d, log2p = %d)", side,
         (long long)n, KQ_MAX_ODD, r->m, r->log2p);
    return false;
  }
  if (!r->signs || !r->q) {
    fail(KQ_EINVAL, "%s rotation: signs or q is NULL", side);
    return false;
  }
  return true;
}

bool ws_ok(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return true;
  if (!ws || ws_bytes < need) {
    fail(KQ_EINVAL, "workspace too small: %zu bytes given, %zu needed", ws ? ws_bytes : size_t(0), need);
    return false;
  }
  return true;
}

}  // namespace

extern "C" {

const char* kq_version(void) { return "kq 0.1.0 (gfx950)"; }

const char* kq_status_string(kq_status s) {
  switch (s) {
    case KQ_OK: return "ok";
    case KQ_EINVAL: return "invalid argument";
    case KQ_ENOTPD: return "matrix not positive definite";
    case KQ_EINFEASIBLE: return "bit budget infeasible";
    case KQ_EDEVICE: return "device error";
    case KQ_EUNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

const char* kq_last_error(void) { return kq::g_error; }

size_t kq_workspace_size(int32_t op, int64_t d0, int64_t d1, int64_t d2) {
  const size_t bad = static_cast<size_t>(-1);
  switch (op) {
    case KQ_OP_ACCUMULATE_COV:
      if (d0 < 0 || d1 < 1 || d1 > kMaxDim) return bad;
      return kq::syrk_workspace(d0, d1);
    case KQ_OP_BIIP:
      if (d0 < 1 || d1 < 1 || d0 > KQ_MAX_ROT_DIM || d1 > KQ_MAX_ROT_DIM) return bad;
      return kq::biip_workspace(d0, d1);
    case KQ_OP_CHOLESKY:
      if (d0 < 1 || d0 > kMaxDim) return bad;
      return kq::chol_workspace(d0);
    case KQ_OP_OBS:
      if (d0 < 1 || d1 < 1 || d2 < 1 || d1 > kMaxDim) return bad;
      return kq::obs_workspace(d0, d1, static_cast<int>(d2));
    case KQ_OP_LOSS:
      if (d0 < 1 || d1 < 1 || d0 > kMaxDim || d1 > kMaxDim) return bad;
      return kq::loss_workspace(d0, d1);
    case KQ_OP_XCOV:
      if (d0 < 0 || d1 < 1 || d1 > kMaxDim) return bad;
      return kq::xcov_workspace(d0, d1);
    case KQ_OP_GPTAQ:
      if (d0 < 1 || d1 < 1 || d0 > kMaxDim || d1 > kMaxDim) return bad;
      return kq::gptaq_workspace(d0, d1);
    case KQ_OP_DECODE:
      if (d0 < 1 || d0 > int64_t(KQ_DECODE_MAX_LAYERS) * KQ_MAX_ROT_DIM || d1 < 1 || d1 > KQ_MAX_ROT_DIM || d2 < 1 ||
          d2 > KQ_DECODE_MAX_TOKENS)
        return bad;
      return kq::decode_workspace(d0, d1, d2);
    default:
      return bad;
  }
}

kq_status kq_accumulate_cov(const uint16_t* a, int64_t rows, int64_t d, int64_t lda, float alpha, float beta,
                            float* h, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 0 || d < 1 || d > kMaxDim) return fail(KQ_EINVAL, "kq_accumulate_cov: bad shape rows=%lld d=%lld",
                                                    (long long)rows, (long long)d);
  if (lda < d) return fail(KQ_EINVAL, "kq_accumulate_cov: lda %lld < d %lld", (long long)lda, (long long)d);
  if (!h || (rows > 0 && !a)) return fail(KQ_EINVAL, "kq_accumulate_cov: NULL pointer");
  if (!ws_ok(ws, ws_bytes, kq::syrk_workspace(rows, d))) return KQ_EINVAL;
  return kq::syrk_run(a, rows, d, lda, alpha, beta, h, ws, kq::as_stream(stream));
}

kq_status kq_accumulate_xcov(const uint16_t* a, const uint16_t* b, int64_t rows, int64_t d, int64_t lda,
                             int64_t ldb, float alpha, float beta, const float* c_in, float* c, void* ws,
                             size_t ws_bytes, void* stream) {
  if (rows < 0 || d < 1 || d > kMaxDim) return fail(KQ_EINVAL, "kq_accumulate_xcov: bad shape rows=%lld d=%lld",
                                                    (long long)rows, (long long)d);
  if (lda < d || ldb < d)
    return fail(KQ_EINVAL, "kq_accumulate_xcov: row pitches %lld, %lld < d %lld", (long long)lda, (long long)ldb,
                (long long)d);
  if (!c || (rows > 0 && (!a || !b))) return fail(KQ_EINVAL, "kq_accumulate_xcov: NULL pointer");
  if (beta != 0.0f && !c_in) return fail(KQ_EINVAL, "kq_accumulate_xcov: beta != 0 needs c_in");
  if (!ws_ok(ws, ws_bytes, kq::xcov_workspace(rows, d))) return KQ_EINVAL;
  return kq::xcov_run(a, b, rows, d, lda, ldb, alpha, beta, c_in, c, ws, kq::as_stream(stream));
}

kq_status kq_biip_transform(float* m, int64_t n, const kq_rot* rot, const double* s, void* ws, size_t ws_bytes,
                            void* stream) {
  if (n < 1 || n > KQ_MAX_ROT_DIM) return fail(KQ_EINVAL, "kq_biip_transform: n = %lld", (long long)n);
  if (!m) return fail(KQ_EINVAL, "kq_biip_transform: NULL pointer");
  if (!rot_ok(rot, n, "input")) return KQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, kq::biip_workspace(n, n))) return KQ_EINVAL;
  return kq::biip_transform_run(m, n, rot, s, ws, kq::as_stream(stream));
}

kq_status kq_gptaq_target(double* w, const float* d2, const float* r, int64_t dout, int64_t din, int32_t* info,
                          void* ws, size_t ws_bytes, void* stream) {
  if (dout < 1 || din < 1 || dout > kMaxDim || din > kMaxDim)
    return fail(KQ_EINVAL, "kq_gptaq_target: shape %lld x %lld", (long long)dout, (long long)din);
  if (!w || !d2 || !r) return fail(KQ_EINVAL, "kq_gptaq_target: NULL pointer");
  if (!ws_ok(ws, ws_bytes, kq::gptaq_workspace(dout, din))) return KQ_EINVAL;
  return kq::gptaq_target_run(w, d2, r, dout, din, info, ws, kq::as_stream(stream));
}

kq_status kq_sensitivity(const float* h_x, int64_t din, const float* h_g, int64_t dout, int32_t mode,
                         double* score, void* stream) {
  if (mode != KQ_SCORE_KRONQ && mode != KQ_SCORE_HX_ONLY) return fail(KQ_EINVAL, "kq_sensitivity: mode %d", mode);
  if (!h_x || !score || din < 1) return fail(KQ_EINVAL, "kq_sensitivity: NULL pointer or din < 1");
  if (mode == KQ_SCORE_KRONQ && (!h_g || dout < 1)) return fail(KQ_EINVAL, "kq_sensitivity: H_G missing");
  return kq::score_run(h_x, din, h_g, dout, mode, score, kq::as_stream(stream));
}

kq_status kq_allocate_bits(const double* score, const int64_t* n_params, int32_t n_layers, const int32_t* choices,
                           int32_t n_choices, int64_t target_millibits, int32_t* bits_out) {
  if (!score || !n_params || !choices || !bits_out) return fail(KQ_EINVAL, "kq_allocate_bits: NULL pointer");
  if (n_layers < 1 || n_choices < 1) return fail(KQ_EINVAL, "kq_allocate_bits: empty problem");
  if (target_millibits < 0) return fail(KQ_EINVAL, "kq_allocate_bits: negative target");
  // a NaN score would make the order below undefined (no strict weak ordering), an infinite
  // one means an overflowed covariance: neither can rank a sub-layer
  for (int32_t l = 0; l < n_layers; ++l)
    if (!std::isfinite(score[l])) return fail(KQ_EINVAL, "kq_allocate_bits: score[%d] is not finite", l);
  std::vector<int32_t> ch(choices, choices + n_choices);
  for (int32_t c : ch)
    if (c < 2 || c > 8) return fail(KQ_EINVAL, "kq_allocate_bits: choice %d outside [2, 8]", c);
  std::sort(ch.begin(), ch.end());
  ch.erase(std::unique(ch.begin(), ch.end()), ch.end());
  __int128 total = 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    if (n_params[l] <= 0) return fail(KQ_EINVAL, "kq_allocate_bits: n_params[%d] <= 0", l);
    total += n_params[l];
  }
  if (total > (__int128(1) << 56)) return fail(KQ_EINVAL, "kq_allocate_bits: parameter count too large");
  const __int128 budget = (__int128(target_millibits) * total) / 1000;
  std::vector<int32_t> bits(n_layers, ch.front());
  __int128 used = __int128(ch.front()) * total;
  if (used > budget) return fail(KQ_EINFEASIBLE, "kq_allocate_bits: budget below min(choices) for all layers");
  std::vector<int32_t> order(n_layers);
  for (int32_t l = 0; l < n_layers; ++l) order[l] = l;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    if (score[x] != score[y]) return score[x] > score[y];
    return x < y;
  });
  for (int32_t l : order) {
    for (auto it = ch.rbegin(); it != ch.rend() && *it > bits[l]; ++it) {
      const __int128 extra = __int128(n_params[l]) * (*it - bits[l]);
      if (used + extra <= budget) {
        used += extra;
        bits[l] = *it;
        break;
      }
    }
  }
  std::memcpy(bits_out, bits.data(), sizeof(int32_t) * n_layers);
  return KQ_OK;
}

kq_status kq_biip_rotate(const void* w, int32_t w_dtype, int64_t dout, int64_t din, double* w_out, float* h_x,
                         float* h_g, const kq_rot* rot_in, const kq_rot* rot_out, uint32_t flags, double* s_x,
                         double* s_g, void* ws, size_t ws_bytes, void* stream) {
  if (flags & ~uint32_t(KQ_BIIP_INPUT | KQ_BIIP_OUTPUT | KQ_BIIP_SCALE | KQ_BIIP_INVERSE))
    return fail(KQ_EINVAL, "kq_biip_rotate: unknown flags 0x%x", flags);
  if (dout < 1 || din < 1 || dout > KQ_MAX_ROT_DIM || din > KQ_MAX_ROT_DIM)
    return fail(KQ_EINVAL, "kq_biip_rotate: shape %lld x %lld outside [1, %d]", (long long)dout, (long long)din,
                KQ_MAX_ROT_DIM);
  if (w_dtype != KQ_BF16 && w_dtype != KQ_F32 && w_dtype != KQ_F64)
    return fail(KQ_EINVAL, "kq_biip_rotate: w_dtype %d", w_dtype);
  if (!w || !w_out || !s_x || !s_g) return fail(KQ_EINVAL, "kq_biip_rotate: NULL pointer");
  const bool inp = flags & KQ_BIIP_INPUT, out = flags & KQ_BIIP_OUTPUT, inverse = flags & KQ_BIIP_INVERSE;
  if (inverse && w_dtype != KQ_F64) return fail(KQ_EINVAL, "kq_biip_rotate: the inverse takes a float64 weight");
  if (inp && !rot_ok(rot_in, din, "input")) return KQ_EINVAL;
  if (out && !rot_ok(rot_out, dout, "output")) return KQ_EINVAL;
  if (!inverse && ((inp && !h_x) || (out && !h_g)))
    return fail(KQ_EINVAL, "kq_biip_rotate: the processed side needs its covariance");
  if (w_out == w) return fail(KQ_EINVAL, "kq_biip_rotate: w_out must not alias w");
  if (!ws_ok(ws, ws_bytes, kq::biip_workspace(dout, din))) return KQ_EINVAL;
  return kq::biip_run(w, w_dtype, dout, din, w_out, h_x, h_g, rot_in, rot_out, flags, s_x, s_g, ws,
                      kq::as_stream(stream));
}

kq_status kq_cholesky_inv(float* h, int64_t d, float damp, int32_t* info, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!h || !info) return fail(KQ_EINVAL, "kq_cholesky_inv: NULL pointer");
  if (d < 1 || d > kMaxDim) return fail(KQ_EINVAL, "kq_cholesky_inv: d = %lld", (long long)d);
  if (!(damp >= 0.0f) || damp > 1e30f) return fail(KQ_EINVAL, "kq_cholesky_inv: damp must be finite and >= 0");
  if (!ws_ok(ws, ws_bytes, kq::chol_workspace(d))) return KQ_EINVAL;
  return kq::chol_run(h, d, damp, info, ws, kq::as_stream(stream));
}

kq_status kq_obs_quantize(double* w, const float* r, int64_t dout, int64_t din, int32_t bits, int32_t group,
                          int32_t block, uint8_t* codes, float* scales, uint8_t* zeros, double* preround, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!w || !r || !codes || !scales || !zeros) return fail(KQ_EINVAL, "kq_obs_quantize: NULL pointer");
  if (reinterpret_cast<uintptr_t>(r) % 16 != 0) return fail(KQ_EINVAL, "kq_obs_quantize: r must be 16-byte aligned");
  if (dout < 1 || din < 1 || din > kMaxDim) return fail(KQ_EINVAL, "kq_obs_quantize: bad shape");
  if (bits < 2 || bits > 8) return fail(KQ_EINVAL, "kq_obs_quantize: bits = %d outside [2, 8]", bits);
  if (block < 1 || din % block != 0)
    return fail(KQ_EINVAL, "kq_obs_quantize: block %d must divide din %lld", block, (long long)din);
  if (group < 0 || (group > 0 && block % group != 0))
    return fail(KQ_EINVAL, "kq_obs_quantize: group %d must be 0 or divide block %d", group, block);
  if (block != 32 && block != 64 && block != 128)
    return fail(KQ_EUNSUPPORTED, "kq_obs_quantize: block %d (supported: 32, 64, 128)", block);
  if (!ws_ok(ws, ws_bytes, kq::obs_workspace(dout, din, block))) return KQ_EINVAL;
  return kq::obs_run(w, r, dout, din, bits, group, block, codes, scales, zeros, preround, ws, kq::as_stream(stream));
}

kq_status kq_kron_loss(const double* w_hat, const void* w, int32_t w_dtype, int64_t dout, int64_t din,
                       const float* h_x, const float* h_g, double* loss, void* ws, size_t ws_bytes, void* stream) {
  if (!w_hat || !w || !h_x || !h_g || !loss) return fail(KQ_EINVAL, "kq_kron_loss: NULL pointer");
  if (dout < 1 || din < 1 || dout > kMaxDim || din > kMaxDim)
    return fail(KQ_EINVAL, "kq_kron_loss: shape %lld x %lld", (long long)dout, (long long)din);
  if (w_dtype != KQ_BF16 && w_dtype != KQ_F32 && w_dtype != KQ_F64)
    return fail(KQ_EINVAL, "kq_kron_loss: w_dtype %d", w_dtype);
  if (!ws_ok(ws, ws_bytes, kq::loss_workspace(dout, din))) return KQ_EINVAL;
  return kq::loss_run(w_hat, w, w_dtype, dout, din, h_x, h_g, loss, ws, kq::as_stream(stream));
}

kq_status kq_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits, uint32_t* packed,
                        void* stream) {
  if (!codes || !packed) return fail(KQ_EINVAL, "kq_pack_codes: NULL pointer");
  if (bits < 2 || bits > 8) return fail(KQ_EINVAL, "kq_pack_codes: bits = %d outside [2, 8]", bits);
  const int per = 32 / kq::container_bits(bits);
  if (rows < 0 || cols < 0 || cols % per != 0)
    return fail(KQ_EINVAL, "kq_pack_codes: %lld columns are not a multiple of %d codes per word", (long long)cols, per);
  return kq::pack_run(codes, rows, cols, bits, packed, kq::as_stream(stream));
}

}  // extern "C"

namespace {

// Argument checks shared by the decode entry points; on success `total` holds the layers' rows.
kq_status decode_check(const kq_decode_layer* layers, int32_t n_layers, int64_t din, int32_t bits, int32_t group,
                       const double* s_x, const kq_rot* rot_in, const float* x, int64_t tokens, int64_t& total) {
  if (!layers || !x) return fail(KQ_EINVAL, "kq_decode_matvec: NULL pointer");
  if (n_layers < 1 || n_layers > KQ_DECODE_MAX_LAYERS)
    return fail(KQ_EINVAL, "kq_decode_matvec_group: %d layers outside [1, %d]", n_layers, KQ_DECODE_MAX_LAYERS);
  if (bits < 2 || bits > 8) return fail(KQ_EINVAL, "kq_decode_matvec: bits = %d outside [2, 8]", bits);
  if (din < 1 || din > KQ_MAX_ROT_DIM || din % 16 != 0)
    return fail(KQ_EINVAL, "kq_decode_matvec: din %lld (a multiple of 16, at most %d)", (long long)din,
                KQ_MAX_ROT_DIM);
  if (group < 0 || (group > 0 && (group % 16 != 0 || din % group != 0)))
    return fail(KQ_EINVAL, "kq_decode_matvec: group %d must be 0 or a multiple of 16 dividing din", group);
  if (tokens < 1 || tokens > KQ_DECODE_MAX_TOKENS)
    return fail(KQ_EINVAL, "kq_decode_matvec: tokens = %lld outside [1, %d]", (long long)tokens,
                KQ_DECODE_MAX_TOKENS);
  if (rot_in && !rot_ok(rot_in, din, "input")) return KQ_EINVAL;
  if (kq::decode_cpl(din, tokens) == 0)
    return fail(KQ_EUNSUPPORTED, "kq_decode_matvec: din %lld with %lld tokens (needs din * tokens <= 16384)",
                (long long)din, (long long)tokens);
  total = 0;
  for (int l = 0; l < n_layers; ++l) {
    const kq_decode_layer& L = layers[l];
    if (!L.packed || !L.scales || !L.zeros || !L.y)
      return fail(KQ_EINVAL, "kq_decode_matvec: NULL pointer in layer %d", l);
    if (L.dout < 1 || L.dout > KQ_MAX_ROT_DIM)
      return fail(KQ_EINVAL, "kq_decode_matvec: layer %d has dout %lld outside [1, %d]", l, (long long)L.dout,
                  KQ_MAX_ROT_DIM);
    if (L.rot_out && !rot_ok(L.rot_out, L.dout, "output")) return KQ_EINVAL;
    if (kq::decode_lds_bytes(L.dout, din, tokens, rot_in || s_x, L.rot_out != nullptr) > 160 * 1024)
      return fail(KQ_EUNSUPPORTED, "kq_decode_matvec: %lld tokens of a %lld x %lld layer exceed LDS",
                  (long long)tokens, (long long)L.dout, (long long)din);
    total += L.dout;
  }
  return KQ_OK;
}

}  // namespace

extern "C" {

kq_status kq_decode_matvec_group(const kq_decode_layer* layers, int32_t n_layers, int64_t din, int32_t bits,
                                 int32_t group, const double* s_x, const kq_rot* rot_in, const float* x,
                                 int64_t tokens, void* ws, size_t ws_bytes, void* stream) {
  int64_t total = 0;
  const kq_status st = decode_check(layers, n_layers, din, bits, group, s_x, rot_in, x, tokens, total);
  if (st != KQ_OK) return st;
  if (!ws_ok(ws, ws_bytes, kq::decode_workspace(total, din, tokens))) return KQ_EINVAL;
  return kq::decode_run(layers, n_layers, din, bits, group, s_x, rot_in, x, tokens, ws, kq::as_stream(stream));
}

kq_status kq_decode_matvec_group_noalloc(const kq_decode_layer* layers, int32_t n_layers, int64_t din, int32_t bits,
                                         int32_t group, const double* s_x, const kq_rot* rot_in, const float* x,
                                         int64_t tokens, void* stream) {
  int64_t total = 0;
  const kq_status st = decode_check(layers, n_layers, din, bits, group, s_x, rot_in, x, tokens, total);
  if (st != KQ_OK) return st;
  const size_t need = kq::decode_workspace(total, din, tokens);
  if (need > size_t(KQ_DECODE_NOALLOC_SCRATCH))
    return fail(KQ_EUNSUPPORTED, "kq_decode_matvec_group_noalloc: needs %zu bytes of scratch, the fixed array holds %d",
                need, KQ_DECODE_NOALLOC_SCRATCH);
  void* ws = nullptr;
  const kq_status sst = kq::decode_static_scratch(&ws);
  if (sst != KQ_OK) return sst;
  return kq::decode_run(layers, n_layers, din, bits, group, s_x, rot_in, x, tokens, ws, kq::as_stream(stream));
}

kq_status kq_decode_matvec(const uint32_t* packed, const float* scales, const uint8_t* zeros, int64_t dout,
                           int64_t din, int32_t bits, int32_t group, const double* s_x, const double* s_g,
                           const kq_rot* rot_in, const kq_rot* rot_out, const float* x, int64_t tokens, float* y,
                           void* ws, size_t ws_bytes, void* stream) {
  const kq_decode_layer layer{packed, scales, zeros, dout, s_g, rot_out, y};
  return kq_decode_matvec_group(&layer, 1, din, bits, group, s_x, rot_in, x, tokens, ws, ws_bytes, stream);
}

}  // extern "C"
