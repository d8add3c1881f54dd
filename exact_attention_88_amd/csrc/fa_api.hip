// C entry points declared in include/fa.h: argument validation (before any
// HIP call), 64-bit stride/alignment analysis, tile lookup and the kernel
// launches on the caller's stream.
#include "../../include/fa.h"

#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "fa_args.h"

namespace {

using fa::BwdArgs;
using fa::FwdArgs;
using fa::T4;

constexpr int64_t kMaxRows = 0x7fffffffLL;

thread_local char g_last_hip[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  if (e == hipErrorInvalidConfiguration) return FA_ERR_SHAPE;
  snprintf(g_last_hip, sizeof(g_last_hip), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return FA_ERR_HIP;
}

bool valid_dtype(int dt) { return dt == FA_F16 || dt == FA_F32 || dt == FA_BF16; }
bool valid_d(int64_t D) { return D == 16 || D == 32 || D == 64 || D == 128; }
int esize(int dt) { return dt == FA_F32 ? 4 : 2; }

bool strides_ok(const int64_t* s) {
  return s != nullptr && s[0] >= 0 && s[1] >= 0 && s[2] >= 0 && s[3] >= 0;
}

// 16-byte vector access is allowed when the d-stride is 1 and every row start
// is 16-byte aligned.
bool vec_ok(const void* p, const int64_t* s, int es) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return s[3] == 1 && (a % 16) == 0 && (s[0] * es) % 16 == 0 && (s[1] * es) % 16 == 0 &&
         (s[2] * es) % 16 == 0;
}

// The kernels need scale * log2(e) > 0: the running max only rises, and
// masked scores are -inf (0 * -inf would be NaN).
bool scale_ok(float scale) { return isfinite(scale) && scale > 0.f; }

T4 mk(const void* p, const int64_t* s) { return T4{p, s[0], s[1], s[2], s[3]}; }

int shape_check(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, int dtype) {
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (!valid_d(D)) return FA_ERR_SHAPE;
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0) return FA_ERR_SHAPE;
  if (Sq > kMaxRows || Sk > kMaxRows || B > kMaxRows || H > kMaxRows) return FA_ERR_SHAPE;
  if (B * H > kMaxRows) return FA_ERR_SHAPE;
  if (B * H * Sq > 0 && Sk == 0) return FA_ERR_SHAPE;
  return FA_OK;
}

// Default tile of a pass: the configuration the offline sweep measured
// fastest for this (dtype, head dim, causal, power-of-two length bucket of
// max(Sq, Sk), clamped to 128..16384) -- "Triton FlashAttention": block sizes
// per power-of-two length bucket -- else the pass's built-in rule.
#include "fa_tile_table.inc"

int tile_default(int pass, int dtype, int D, int64_t Sq, int64_t Sk, int causal) {
  int (*rule)(int, int, int64_t, int64_t, int) = pass == FA_PASS_FWD      ? fa::fwd_tile_default
                                               : pass == FA_PASS_BWD_DKDV ? fa::dkdv_tile_default
                                                                          : fa::dq_tile_default;
  int (*count)(int, int) = pass == FA_PASS_FWD      ? fa::fwd_tile_count
                           : pass == FA_PASS_BWD_DKDV ? fa::dkdv_tile_count
                                                      : fa::dq_tile_count;
  const int di = D == 16 ? 0 : D == 32 ? 1 : D == 64 ? 2 : 3;
  const int64_t len = Sq > Sk ? Sq : Sk;
  int bi = 0;
  while (bi < 7 && ((int64_t)128 << bi) < len) ++bi;
  const int id = kSweptTiles[pass][dtype][di][causal ? 1 : 0][bi];
  if (id >= 0 && id < count(dtype, D)) return id;
  return rule(dtype, D, Sq, Sk, causal);
}

int fwd_impl(int tile, const void* q, const int64_t* qs, const void* k, const int64_t* ks,
             const void* v, const int64_t* vs, int64_t B, int64_t H, int64_t Sq, int64_t Sk,
             int64_t D, int causal, float scale, int dtype, void* out, const int64_t* os,
             float* lse, void* stream) {
  int st = shape_check(B, H, Sq, Sk, D, dtype);
  if (st != FA_OK) return st;
  if (causal < 0 || causal > 2) return FA_ERR_CAUSAL;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  if (B * H * Sq == 0) return FA_OK;
  if (!q || !k || !v || !out || !lse) return FA_ERR_NULL;
  if (!qs || !ks || !vs || !os) return FA_ERR_NULL;
  if (!strides_ok(qs) || !strides_ok(ks) || !strides_ok(vs) || !strides_ok(os))
    return FA_ERR_STRIDE;
  if (out == q || out == k || out == v || (const void*)lse == q || (const void*)lse == k ||
      (const void*)lse == v || (void*)lse == out)
    return FA_ERR_ALIAS;
  const int dt = dtype;
  const int d = (int)D;
  if (tile < 0) tile = tile_default(FA_PASS_FWD, dt, d, Sq, Sk, causal);
  if (tile >= fa::fwd_tile_count(dt, d)) return FA_ERR_TILE;
  const int es = esize(dt);
  FwdArgs a;
  a.q = mk(q, qs);
  a.k = mk(k, ks);
  a.v = mk(v, vs);
  a.o = mk(out, os);
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.Sq = (int)Sq;
  a.Sk = (int)Sk;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.vec = (vec_ok(q, qs, es) ? fa::VEC_Q : 0) | (vec_ok(k, ks, es) ? fa::VEC_K : 0) |
          (vec_ok(v, vs, es) ? fa::VEC_V : 0) | (vec_ok(out, os, es) ? fa::VEC_O : 0);
  a.coff = causal == 2 ? (int)(Sk - Sq) : 0;
  return hip_status(fa::launch_fwd(a, dt, d, causal ? 1 : 0, tile, (hipStream_t)stream));
}

// stage: -1 = all three kernels; 0 = preprocess; 1 = dK/dV; 2 = dQ;
// -2 = validate the arguments and launch nothing.
int bwd_impl(int stage, int tile_kv, int tile_q, const void* q, const int64_t* qs, const void* k,
             const int64_t* ks, const void* v, const int64_t* vs, const void* o,
             const int64_t* os, const void* dout, const int64_t* dos, const float* lse,
             int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, int causal, float scale,
             int dtype, float* delta, void* dq, const int64_t* dqs, void* dk, const int64_t* dks,
             void* dv, const int64_t* dvs, void* stream) {
  int st = shape_check(B, H, Sq, Sk, D, dtype);
  if (st != FA_OK) return st;
  if (causal < 0 || causal > 2) return FA_ERR_CAUSAL;
  if (!scale_ok(scale)) return FA_ERR_SCALE;
  if (B * H == 0 || (Sq == 0 && Sk == 0)) return FA_OK;
  const bool has_q = Sq > 0;
  if (!k || !v || !dk || !dv || !ks || !vs || !dks || !dvs) return FA_ERR_NULL;
  if (has_q && (!q || !o || !dout || !lse || !delta || !dq || !qs || !os || !dos || !dqs))
    return FA_ERR_NULL;
  if (!strides_ok(ks) || !strides_ok(vs) || !strides_ok(dks) || !strides_ok(dvs))
    return FA_ERR_STRIDE;
  if (has_q && (!strides_ok(qs) || !strides_ok(os) || !strides_ok(dos) || !strides_ok(dqs)))
    return FA_ERR_STRIDE;
  {
    const void* ins[6] = {q, k, v, o, dout, lse};
    const void* outs[4] = {delta, dq, dk, dv};
    for (int i = 0; i < 4; ++i) {
      if (!outs[i]) continue;
      for (int j = 0; j < 6; ++j)
        if (ins[j] && outs[i] == ins[j]) return FA_ERR_ALIAS;
      for (int j = i + 1; j < 4; ++j)
        if (outs[j] && outs[i] == outs[j]) return FA_ERR_ALIAS;
    }
  }
  const int dt = dtype;
  const int d = (int)D;
  if (tile_kv < 0) tile_kv = tile_default(FA_PASS_BWD_DKDV, dt, d, Sq, Sk, causal);
  if (tile_q < 0) tile_q = tile_default(FA_PASS_BWD_DQ, dt, d, Sq, Sk, causal);
  if (tile_kv >= fa::dkdv_tile_count(dt, d) || tile_q >= fa::dq_tile_count(dt, d))
    return FA_ERR_TILE;
  static const int64_t zs[4] = {0, 0, 0, 1};
  const int es = esize(dt);
  BwdArgs a;
  a.q = mk(q, has_q ? qs : zs);
  a.k = mk(k, ks);
  a.v = mk(v, vs);
  a.o = mk(o, has_q ? os : zs);
  a.dout = mk(dout, has_q ? dos : zs);
  a.dq = mk(dq, has_q ? dqs : zs);
  a.dk = mk(dk, dks);
  a.dv = mk(dv, dvs);
  a.lse = lse;
  a.delta = delta;
  a.B = (int)B;
  a.H = (int)H;
  a.Sq = (int)Sq;
  a.Sk = (int)Sk;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  int vec = (vec_ok(k, ks, es) ? fa::VEC_K : 0) | (vec_ok(v, vs, es) ? fa::VEC_V : 0) |
            (vec_ok(dk, dks, es) ? fa::VEC_DK : 0) | (vec_ok(dv, dvs, es) ? fa::VEC_DV : 0);
  if (has_q)
    vec |= (vec_ok(q, qs, es) ? fa::VEC_Q : 0) | (vec_ok(o, os, es) ? fa::VEC_O : 0) |
           (vec_ok(dout, dos, es) ? fa::VEC_DO : 0) | (vec_ok(dq, dqs, es) ? fa::VEC_DQ : 0);
  a.vec = vec;
  a.coff = causal == 2 ? (int)(Sk - Sq) : 0;
  // delta = rowsum(dO o O) comes from its own kernel (stage 0) or, where the
  // chosen dQ kernel can form it from the rows it holds, from the dQ kernel
  // (stage 2), which then runs first; the dK/dV kernel (stage 1) reads it.
  a.fuse_delta = has_q && fa::dq_can_fuse_delta(a, dt, d, tile_q) ? 1 : 0;
  if (stage == -2) return FA_OK;  // validation only (fa_bwd_noalloc's pre-check)
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (has_q && !a.fuse_delta && (stage < 0 || stage == 0)) e = fa::launch_bwd_pre(a, dt, d, s);
  if (e == hipSuccess && has_q && (stage < 0 || stage == 2))
    e = fa::launch_dq(a, dt, d, causal ? 1 : 0, tile_q, s);
  if (e == hipSuccess && Sk > 0 && (stage < 0 || stage == 1))
    e = fa::launch_dkdv(a, dt, d, causal ? 1 : 0, tile_kv, s);
  return hip_status(e);
}

// Scratch of the allocation-free backward (fa_bwd_noalloc): the delta
// workspace, one array per device in the library's own device globals, so
// the call allocates nothing.  Host code never passes `scratch` itself to a
// kernel (in host code the name is a host-side stand-in, not the device
// array): each device's address comes from hipGetSymbolAddress, taken once
// per device on its first call with that device current.
constexpr int64_t kScratchRows = (int64_t)1 << 22;  // delta floats: B*H*Sq limit, 16 MiB
__device__ __attribute__((aligned(256))) float scratch[kScratchRows];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

// This device's scratch address (FA_OK) or a fa_status.
int scratch_for_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return FA_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(const void* q, const int64_t q_strides[4], const void* k,
                   const int64_t k_strides[4], const void* v, const int64_t v_strides[4],
                   const void* o, const int64_t o_strides[4], const void* dout,
                   const int64_t dout_strides[4], const float* lse, int64_t B, int64_t H,
                   int64_t Sq, int64_t Sk, int64_t D, int causal, float scale, int dtype,
                   void* dq, const int64_t dq_strides[4], void* dk, const int64_t dk_strides[4],
                   void* dv, const int64_t dv_strides[4], void* stream) {
  // Argument checks first (no HIP call): fa_bwd's own, with a stand-in
  // non-null workspace pointer that is never dereferenced by a rejected
  // call, plus the scratch limit.
  const int st = shape_check(B, H, Sq, Sk, D, dtype);
  if (st != FA_OK) return st;
  if (B > 0 && H > 0 && Sq > 0 && B * H * Sq > kScratchRows) return FA_ERR_WORKSPACE;
  float* ws = nullptr;
  if (B * H * Sq > 0 && Sk > 0) {
    // Validate everything fa_bwd validates before touching the device.
    const int pre = bwd_impl(-2, -1, -1, q, q_strides, k, k_strides, v, v_strides, o, o_strides,
                             dout, dout_strides, lse, B, H, Sq, Sk, D, causal, scale, dtype,
                             reinterpret_cast<float*>(uintptr_t(1)), dq, dq_strides, dk,
                             dk_strides, dv, dv_strides, stream);
    if (pre != FA_OK) return pre;
    const int sst = scratch_for_current_device(&ws);
    if (sst != FA_OK) return sst;
  }
  return bwd_impl(-1, -1, -1, q, q_strides, k, k_strides, v, v_strides, o, o_strides, dout,
                  dout_strides, lse, B, H, Sq, Sk, D, causal, scale, dtype, ws, dq, dq_strides,
                  dk, dk_strides, dv, dv_strides, stream);
}

int fa_fwd(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
           const void* v, const int64_t v_strides[4], int64_t B, int64_t H, int64_t Sq,
           int64_t Sk, int64_t D, int causal, float scale, int dtype, void* out,
           const int64_t out_strides[4], float* lse, void* stream) {
  return fwd_impl(-1, q, q_strides, k, k_strides, v, v_strides, B, H, Sq, Sk, D, causal, scale,
                  dtype, out, out_strides, lse, stream);
}

int fa_fwd_tile(int tile_id, const void* q, const int64_t q_strides[4], const void* k,
                const int64_t k_strides[4], const void* v, const int64_t v_strides[4],
                int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D, int causal,
                float scale, int dtype, void* out, const int64_t out_strides[4], float* lse,
                void* stream) {
  if (tile_id < -1) return FA_ERR_TILE;
  return fwd_impl(tile_id, q, q_strides, k, k_strides, v, v_strides, B, H, Sq, Sk, D, causal,
                  scale, dtype, out, out_strides, lse, stream);
}

int fa_bwd(const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4],
           const void* v, const int64_t v_strides[4], const void* o, const int64_t o_strides[4],
           const void* dout, const int64_t dout_strides[4], const float* lse, int64_t B,
           int64_t H, int64_t Sq, int64_t Sk, int64_t D, int causal, float scale, int dtype,
           float* delta_ws, void* dq, const int64_t dq_strides[4], void* dk,
           const int64_t dk_strides[4], void* dv, const int64_t dv_strides[4], void* stream) {
  return bwd_impl(-1, -1, -1, q, q_strides, k, k_strides, v, v_strides, o, o_strides, dout,
                  dout_strides, lse, B, H, Sq, Sk, D, causal, scale, dtype, delta_ws, dq,
                  dq_strides, dk, dk_strides, dv, dv_strides, stream);
}

int fa_bwd_tile(int dkdv_tile_id, int dq_tile_id, const void* q, const int64_t q_strides[4],
                const void* k, const int64_t k_strides[4], const void* v,
                const int64_t v_strides[4], const void* o, const int64_t o_strides[4],
                const void* dout, const int64_t dout_strides[4], const float* lse, int64_t B,
                int64_t H, int64_t Sq, int64_t Sk, int64_t D, int causal, float scale,
                int dtype, float* delta_ws, void* dq, const int64_t dq_strides[4], void* dk,
                const int64_t dk_strides[4], void* dv, const int64_t dv_strides[4],
                void* stream) {
  if (dkdv_tile_id < -1 || dq_tile_id < -1) return FA_ERR_TILE;
  return bwd_impl(-1, dkdv_tile_id, dq_tile_id, q, q_strides, k, k_strides, v, v_strides, o,
                  o_strides, dout, dout_strides, lse, B, H, Sq, Sk, D, causal, scale, dtype,
                  delta_ws, dq, dq_strides, dk, dk_strides, dv, dv_strides, stream);
}

int fa_bwd_stage(int stage, int tile_id, const void* q, const int64_t q_strides[4],
                 const void* k, const int64_t k_strides[4], const void* v,
                 const int64_t v_strides[4], const void* o, const int64_t o_strides[4],
                 const void* dout, const int64_t dout_strides[4], const float* lse, int64_t B,
                 int64_t H, int64_t Sq, int64_t Sk, int64_t D, int causal, float scale,
                 int dtype, float* delta_ws, void* dq, const int64_t dq_strides[4], void* dk,
                 const int64_t dk_strides[4], void* dv, const int64_t dv_strides[4],
                 void* stream) {
  if (stage < 0 || stage > 2) return FA_ERR_TILE;
  if (tile_id < -1) return FA_ERR_TILE;
  // Stages 0 and 2 take the dQ tile: it decides whether delta comes from its
  // own kernel (stage 0) or from the dQ kernel (stage 2).
  return bwd_impl(stage, stage == 1 ? tile_id : -1, stage != 1 ? tile_id : -1, q, q_strides, k,
                  k_strides, v, v_strides, o, o_strides, dout, dout_strides, lse, B, H, Sq, Sk,
                  D, causal, scale, dtype, delta_ws, dq, dq_strides, dk, dk_strides, dv,
                  dv_strides, stream);
}

int fa_tile_count(int pass, int dtype, int64_t D) {
  if (!valid_dtype(dtype) || !valid_d(D)) return 0;
  switch (pass) {
    case FA_PASS_FWD: return fa::fwd_tile_count(dtype, (int)D);
    case FA_PASS_BWD_DKDV: return fa::dkdv_tile_count(dtype, (int)D);
    case FA_PASS_BWD_DQ: return fa::dq_tile_count(dtype, (int)D);
  }
  return 0;
}

int fa_tile_info(int pass, int dtype, int64_t D, int tile_id, int64_t info[4]) {
  if (!info) return FA_ERR_NULL;
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (!valid_d(D)) return FA_ERR_SHAPE;
  const fa::TileCfg* t = nullptr;
  switch (pass) {
    case FA_PASS_FWD: t = fa::fwd_tile(dtype, (int)D, tile_id); break;
    case FA_PASS_BWD_DKDV: t = fa::dkdv_tile(dtype, (int)D, tile_id); break;
    case FA_PASS_BWD_DQ: t = fa::dq_tile(dtype, (int)D, tile_id); break;
    default: return FA_ERR_TILE;
  }
  if (!t) return FA_ERR_TILE;
  info[0] = t->bm;
  info[1] = t->bn;
  info[2] = t->waves;
  info[3] = t->lds;
  return FA_OK;
}

int fa_tile_default(int pass, int dtype, int64_t D, int64_t Sq, int64_t Sk, int causal) {
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (!valid_d(D)) return FA_ERR_SHAPE;
  if (pass < FA_PASS_FWD || pass > FA_PASS_BWD_DQ) return FA_ERR_TILE;
  if (causal < 0 || causal > 2) return FA_ERR_CAUSAL;
  if (Sq < 0 || Sk < 0) return FA_ERR_SHAPE;
  return tile_default(pass, dtype, (int)D, Sq, Sk, causal);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: unsupported or inconsistent sizes";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype";
    case FA_ERR_STRIDE: return "FA_ERR_STRIDE: negative stride";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: an output aliases an input or another output";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error at launch";
    case FA_ERR_TILE: return "FA_ERR_TILE: tile id out of range";
    case FA_ERR_CAUSAL: return "FA_ERR_CAUSAL: causal must be 0, 1 (top-left) or 2 (bottom-right)";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_WORKSPACE:
      return "FA_ERR_WORKSPACE: B*H*Sq exceeds the allocation-free entry point's scratch (2^22 rows)";
  }
  return "unknown fa_status";
}

const char* fa_last_hip_error(void) { return g_last_hip; }

#define FA_STR2(x) #x
#define FA_STR(x) FA_STR2(x)
const char* fa_version(void) {
  return "fa-mi355x 0.2 gfx950; HIP " FA_STR(HIP_VERSION_MAJOR) "." FA_STR(HIP_VERSION_MINOR) "." FA_STR(
      HIP_VERSION_PATCH) "; " __VERSION__;
}

}  // extern "C"
