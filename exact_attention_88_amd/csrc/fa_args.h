// Kernel argument blocks and launcher declarations shared by the host entry
// points (fa_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// A logical [B, H, S, D] tensor: base pointer and element strides.
struct T4 {
  const void* p;
  int64_t sb, sh, ss, sd;
};

enum : int {
  VEC_Q = 1, VEC_K = 2, VEC_V = 4, VEC_O = 8, VEC_DO = 16, VEC_DQ = 32, VEC_DK = 64, VEC_DV = 128
};

struct FwdArgs {
  T4 q, k, v, o;
  float* lse;
  int B, H, Sq, Sk;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int vec;           // VEC_* bits: 16-byte vector access allowed per tensor
  int coff;          // causal: query i sees keys j <= i + coff (0 top-left, Sk - Sq bottom-right)
};

struct BwdArgs {
  T4 q, k, v, o, dout, dq, dk, dv;
  const float* lse;
  float* delta;
  int B, H, Sq, Sk;
  float scale;       // softmax scale (applied to dq, dk)
  float scale_log2;  // scale * log2(e)
  int vec;
  int coff;          // causal: query i sees keys j <= i + coff (0 top-left, Sk - Sq bottom-right)
  int fuse_delta;    // the dQ kernel computes delta = rowsum(dO o O) itself and writes it
};

struct TileCfg {
  int bm;     // query rows per workgroup (forward, dq) / per inner step (dk/dv)
  int bn;     // keys per inner step (forward, dq) / per workgroup (dk/dv)
  int waves;  // wavefronts per workgroup
  int lds;    // static LDS bytes
};

// Element dtypes (the fa_dtype values): 0 = f16, 1 = f32, 2 = bf16.  The two
// 16-bit types share tile tables and kernel shapes.
constexpr int table_dt(int dtype) { return dtype == 1 ? 1 : 0; }
constexpr int elem_size(int dtype) { return dtype == 1 ? 4 : 2; }

// Per-pass tile tables (index = tile id) for a dtype and head dim; count
// returns the number of entries.
int fwd_tile_count(int dtype, int D);
const TileCfg* fwd_tile(int dtype, int D, int id);
int fwd_tile_default(int dtype, int D, int64_t Sq, int64_t Sk, int causal);
hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, int causal, int tile, hipStream_t s);

// Tuned 16-bit (fp16 and bf16) forward for head dims 128 and 64
// (fa_fwd_f16.hip); fwd_fast_runs tells whether launch_fwd_fast can take
// these arguments (else a generic entry runs).
int fwd_fast_variants(int D);
TileCfg fwd_fast_cfg(int variant, int D);
bool fwd_fast_runs(const FwdArgs& a, int dtype, int D);
hipError_t launch_fwd_fast(const FwdArgs& a, int variant, int dtype, int D, int causal, hipStream_t s);

int dkdv_tile_count(int dtype, int D);
const TileCfg* dkdv_tile(int dtype, int D, int id);
int dkdv_tile_default(int dtype, int D, int64_t Sq, int64_t Sk, int causal);
hipError_t launch_dkdv(const BwdArgs& a, int dtype, int D, int causal, int tile, hipStream_t s);

int dq_tile_count(int dtype, int D);
const TileCfg* dq_tile(int dtype, int D, int id);
int dq_tile_default(int dtype, int D, int64_t Sq, int64_t Sk, int causal);
hipError_t launch_dq(const BwdArgs& a, int dtype, int D, int causal, int tile, hipStream_t s);
// Whether launch_dq with this tile runs a kernel that can compute delta itself
// (the buffer-load dQ kernel, which holds each query row's dO and reads its O
// row), so that the separate rowsum(dO o O) kernel is not needed.
bool dq_can_fuse_delta(const BwdArgs& a, int dtype, int D, int tile);

hipError_t launch_bwd_pre(const BwdArgs& a, int dtype, int D, hipStream_t s);

// Tuned 16-bit (fp16, bf16) backward kernels for head dims 128 and 64
// (fa_bwd_f16.hip); *_fast_runs tells whether the launcher can take these
// arguments (else a generic entry runs).
int dq_fast_variants(int D);
TileCfg dq_fast_cfg(int variant, int D);
bool dq_fast_runs(const BwdArgs& a, int dtype, int D);
hipError_t launch_dq_fast(const BwdArgs& a, int variant, int dtype, int D, int causal, hipStream_t s);
bool dq_fast_fuses_delta(const BwdArgs& a, int variant, int dtype, int D);
int dkdv_fast_variants(int D);
TileCfg dkdv_fast_cfg(int variant, int D);
bool dkdv_fast_runs(const BwdArgs& a, int dtype, int D);
hipError_t launch_dkdv_fast(const BwdArgs& a, int variant, int dtype, int D, int causal, hipStream_t s);
// dK/dV with each 32-key slice split over a score wave and an accumulate wave
// (fa_bwd_split.hip).
bool dkdv_split_fits(const BwdArgs& a, int esize);
int dkdv_split_lds();
hipError_t launch_dkdv_split(const BwdArgs& a, int dtype, int causal, hipStream_t s);

}  // namespace fa
