// Shared device helpers for the gfx950 attention kernels: MFMA wrappers, lane
// layouts, strided tile loaders and the transposed LDS fragment reads.
//
// Lane layouts of the 32x32 MFMAs used here (one wave64, g = lane/32,
// c = lane%32; checked on gfx950):
//   A (32 x K):  lane holds A[c][g*KPL + e], e < KPL
//   B (K x 32):  lane holds B[g*KPL + e][c]
//   C (32 x 32): lane holds, in register r, C[crow(r, g)][c]
//                with crow(r, g) = (r/4)*8 + g*4 + r%4
// KPL = 8, K = 16 for v_mfma_f32_32x32x16_f16 and v_mfma_f32_32x32x16_bf16,
// and KPL = 1, K = 2 for the full-precision v_mfma_f32_32x32x2f32.
//
// The accumulator layout puts one column (a fixed query or key) in each lane
// and spreads the other index over registers.  Feeding a C tile back as the
// B operand of the next product therefore needs no data movement when the
// contraction slots are labelled by crow(): slot e of k-step t stands for
// index crow(t*KPL + e, g) of the 32-block.  The A operand of that product
// must use the same labelling, which is what frag_tr() reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 half_t;
typedef __bf16 bf16_t;
template <class T> using V8 = T __attribute__((ext_vector_type(8)));
template <class T> using V4 = T __attribute__((ext_vector_type(4)));
typedef V8<half_t> h8;
typedef V4<half_t> h4;
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <class T> struct Mfma;

template <> struct Mfma<half_t> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef h8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<bf16_t> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef V8<bf16_t> frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Workgroup -> (block rank within its (b,h), b*h).  Workgroups go out to the
// 8 XCDs round robin (id % 8); each (b,h)'s nb blocks stay on one XCD so that
// its L2 serves their shared K/V (or Q/dO) stream.  With by_rank, and whole
// heads on every XCD, an XCD's heads go out in groups of kHeadGroup, and a
// group's workgroups rank by rank across its heads (rank 0 of every head of
// the group first) rather than head by head: the causal kernels give rank 0
// the most work, so this is longest-first scheduling within the group and the
// launch does not end on the long blocks of the XCD's last head, while at
// most a group's heads' streams share the XCD's L2 at a time (rank by rank
// across all of an XCD's heads, at S = 512 and 1024 with 32 and more heads
// an XCD, the dQ and dK/dV kernels ran 5-10 % slower: the heads' streams no
// longer fit its L2).  The causal forward, dQ and dK/dV kernels take it.
constexpr int kHeadGroup = 4;

__device__ __forceinline__ void xcd_block(int nb, bool by_rank, int& rank, int& bh) {
  const int n = gridDim.x, id = blockIdx.x;
  int L = id;
  if (n % 8 == 0) {
    const int per = n / 8, x = id % 8, slot = id / 8;
    if (by_rank && per % nb == 0) {
      const int hx = per / nb;
      const int gh = hx % kHeadGroup == 0 ? kHeadGroup : hx;
      const int grp = slot / (gh * nb), s2 = slot - grp * gh * nb;
      rank = s2 / gh;
      bh = x * hx + grp * gh + s2 % gh;
      return;
    }
    L = x * per + slot;
  }
  rank = L % nb;
  bh = L / nb;
}

__device__ __forceinline__ int crow(int r, int g) { return (r >> 2) * 8 + g * 4 + (r & 3); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Row stride (elements) of a row-major [rows][D] tile in LDS: at least 32
// columns so that transposed reads of a 32-wide column block stay inside the
// row, plus a 16-byte pad.
template <class T, int D> struct LdsRow {
  static constexpr int W = D < 32 ? 32 : D;
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int LS = W + PAD;
};

// ---------------------------------------------------------------------------
// Global -> LDS tile load: rows [row0, row0 + ROWS) of a strided [S][D]
// matrix into lds[r * LS + col].  Rows >= nrows are zero-filled.  `vec`
// selects 16-byte loads (unit d-stride, 16-byte aligned rows).
template <class T, int ROWS, int D, int LS, int NT>
__device__ __forceinline__ void load_tile(T* __restrict__ lds, const T* __restrict__ base,
                                          int64_t ss, int64_t sd, int row0, int nrows,
                                          bool vec) {
  constexpr int CH = 16 / (int)sizeof(T);
  constexpr int CPR = D / CH;
  constexpr int TOTAL = ROWS * CPR;
#pragma unroll
  for (int it = 0; it < (TOTAL + NT - 1) / NT; ++it) {
    const int c = it * NT + (int)threadIdx.x;
    if (TOTAL % NT == 0 || c < TOTAL) {
      const int r = c / CPR, col = (c % CPR) * CH;
      const int row = row0 + r;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (row < nrows) {
        const T* src = base + (int64_t)row * ss;
        if (vec) {
          val = *reinterpret_cast<const uint4*>(src + col);
        } else {
          T tmp[CH];
#pragma unroll
          for (int e = 0; e < CH; ++e) tmp[e] = src[(int64_t)(col + e) * sd];
          __builtin_memcpy(&val, tmp, 16);
        }
      }
      *reinterpret_cast<uint4*>(lds + r * LS + col) = val;
    }
  }
}

// The same tile load split in two, for double buffering: load() issues the
// global reads of rows [row0, row0 + ROWS) into registers (rows >= nrows give
// zeros), store() writes them to LDS later, so the reads of tile t+1 are in
// flight while tile t is computed.
template <class T, int ROWS, int D, int LS, int NT>
struct TileStage {
  static constexpr int CH = 16 / (int)sizeof(T);
  static constexpr int CPR = D / CH;
  static constexpr int TOTAL = ROWS * CPR;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  uint4 r[PER];

  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ss, int64_t sd, int row0,
                                       int nrows, bool vec) {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = it * NT + (int)threadIdx.x;
      r[it] = make_uint4(0u, 0u, 0u, 0u);
      if (TOTAL % NT == 0 || c < TOTAL) {
        const int row = row0 + c / CPR, col = (c % CPR) * CH;
        if (row < nrows) {
          const T* src = base + (int64_t)row * ss;
          if (vec) {
            r[it] = *reinterpret_cast<const uint4*>(src + col);
          } else {
            T tmp[CH];
#pragma unroll
            for (int e = 0; e < CH; ++e) tmp[e] = src[(int64_t)(col + e) * sd];
            __builtin_memcpy(&r[it], tmp, 16);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ lds) const {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = it * NT + (int)threadIdx.x;
      if (TOTAL % NT == 0 || c < TOTAL)
        *reinterpret_cast<uint4*>(lds + (c / CPR) * LS + (c % CPR) * CH) = r[it];
    }
  }
};

// Register fragments of rows of a strided [S][D] matrix, laid out as the B
// operand of X^T (or the A operand of X): lane holds
// X[row][ks*KSTEP + g*KPL + e] in frag[ks].  Rows >= nrows give zeros.
template <class T, int D>
__device__ __forceinline__ void load_row_frags(typename Mfma<T>::frag* f, const T* __restrict__ base,
                                               int64_t ss, int64_t sd, int row, int nrows,
                                               bool vec) {
  typedef Mfma<T> M;
  constexpr int NKS = D / M::KSTEP;
  const int g = (threadIdx.x & 63) >> 5;
  if (row >= nrows) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) f[ks] = typename M::frag{};
    return;
  }
  const T* src = base + (int64_t)row * ss;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int col = ks * M::KSTEP + g * M::KPL;
    if constexpr (sizeof(T) == 2) {
      if (vec) {
        f[ks] = *reinterpret_cast<const typename M::frag*>(src + col);
      } else {
        typename M::frag t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = src[(int64_t)(col + e) * sd];
        f[ks] = t;
      }
    } else {
      f[ks] = src[(int64_t)col * sd];
    }
  }
}

// A/B fragment of a row-major LDS tile, untransposed: lane holds
// lds[(rbase + c) * LS + cbase + g*KPL + e].
template <class T, int LS>
__device__ __forceinline__ typename Mfma<T>::frag frag_rows(const T* lds, int rbase, int cbase) {
  const int lane = threadIdx.x & 63, g = lane >> 5, c = lane & 31;
  const T* p = lds + (rbase + c) * LS + cbase + g * Mfma<T>::KPL;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const typename Mfma<T>::frag*>(p);
  } else {
    return *p;
  }
}

// 32x32 block C = X[rbase.., :] * B over the head dim, X read row-wise from
// LDS (frag_rows) and B from registers (bf[ks], ks < D/KSTEP).  For fp32 the
// contraction is split into chains of 16 head-dim elements whose sums are
// combined by compensated (Kahan) summation, which keeps the rounding of long
// dot products of large scores (peaked softmax) well inside fp32 tolerances
// with only two partial sums live; every fp32 kernel forms its scores this
// way, so the backward's recomputed scores match the forward's bit for bit
// and their rounding cancels in P = exp(S - LSE).  fp16 uses one chain.
template <class T, int D, int LS>
__device__ __forceinline__ f32x16 dot_block(const T* lds, int rbase,
                                            const typename Mfma<T>::frag* bf) {
  typedef Mfma<T> M;
  constexpr int NKS = D / M::KSTEP;
  if constexpr (sizeof(T) == 2) {
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      acc = M::mma(frag_rows<T, LS>(lds, rbase, ks * M::KSTEP), bf[ks], acc);
    return acc;
  } else {
    constexpr int CHAIN = 8;  // MFMA steps (16 elements) per partial sum
    constexpr int NCH = NKS / CHAIN;  // 1, 2, 4 or 8
    auto chain = [&](int c) {
      f32x16 x = zero16();
#pragma unroll
      for (int k = 0; k < CHAIN; ++k) {
        const int ks = c * CHAIN + k;
        x = M::mma(frag_rows<T, LS>(lds, rbase, ks * M::KSTEP), bf[ks], x);
      }
      return x;
    };
    f32x16 acc = chain(0), err = zero16();
#pragma unroll
    for (int c = 1; c < NCH; ++c) {
      const f32x16 x = chain(c);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y = x[r] - err[r];
        const float t = acc[r] + y;
        err[r] = (t - acc[r]) - y;
        acc[r] = t;
      }
    }
    return acc;
  }
}

// A fragment of the TRANSPOSE of a row-major LDS tile X[rows][cols], for
// k-step t of a 32-row block starting at rbase, output column block cbase:
// lane (c, g) holds, for slot e, X[rbase + crow(t*KPL + e, g)][cbase + c].
// For half precision this is two ds_read_b64_tr_b16 reads: within each
// group of 16 lanes, lane j points at 4 consecutive elements of row j/4 and
// receives column j of the 4 rows.
template <class T, int LS>
__device__ __forceinline__ typename Mfma<T>::frag frag_tr(const T* lds, int rbase, int t,
                                                          int cbase) {
  const int lane = threadIdx.x & 63, g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    const int j = lane & 15;
    const int col = cbase + ((lane >> 4) & 1) * 16 + (j & 3) * 4;
    const int row = rbase + t * 16 + g * 4 + (j >> 2);
    typedef __attribute__((address_space(3))) s4 lds_s4;
    const T* p0 = lds + row * LS + col;
    const T* p1 = p0 + 8 * LS;
    s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
    s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p1));
    V4<T> ah = __builtin_bit_cast(V4<T>, a), bh = __builtin_bit_cast(V4<T>, b);
    typename Mfma<T>::frag r;
    r[0] = ah[0]; r[1] = ah[1]; r[2] = ah[2]; r[3] = ah[3];
    r[4] = bh[0]; r[5] = bh[1]; r[6] = bh[2]; r[7] = bh[3];
    return r;
  } else {
    const int c = lane & 31;
    return lds[(rbase + crow(t, g)) * LS + cbase + c];
  }
}

// B fragment built from accumulator registers t*KPL .. t*KPL+KPL-1 of a 32x32
// C tile, rounded to T (round to nearest even).
template <class T>
__device__ __forceinline__ typename Mfma<T>::frag frag_from_acc(const f32x16& acc, int t) {
  if constexpr (sizeof(T) == 2) {
    typename Mfma<T>::frag r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (T)acc[t * 8 + e];
    return r;
  } else {
    return acc[t];
  }
}

// Store 4 consecutive fp32 values v[0..3] to a strided row at column col
// (columns >= D are dropped), converting to T.
template <class T, int D>
__device__ __forceinline__ void store4(T* __restrict__ rowp, int64_t sd, int col, const float* v,
                                      bool vec) {
  if (col >= D) return;
  if constexpr (sizeof(T) == 2) {
    if (vec) {
      V4<T> h;
      h[0] = (T)v[0]; h[1] = (T)v[1]; h[2] = (T)v[2]; h[3] = (T)v[3];
      *reinterpret_cast<V4<T>*>(rowp + col) = h;
      return;
    }
  } else {
    if (vec) {
      *reinterpret_cast<float4*>(rowp + col) = make_float4(v[0], v[1], v[2], v[3]);
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) rowp[(int64_t)(col + e) * sd] = (T)v[e];
}

}  // namespace fa
