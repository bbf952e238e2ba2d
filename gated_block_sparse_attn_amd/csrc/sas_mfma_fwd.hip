// Matrix-core (MFMA) forward of SAS gated block-sparse attention, bf16 inputs,
// fp32 accumulation, block b = 64 tokens, head_dim D = 128, on gfx950.
//
// Computes Sec. 4.3 Eq. 9 of the SAS paper (arXiv 2609.13141) in the
// streaming form of its App. E forward (Alg. 3): for query block i the
// current block comes first (unit gate, causal), then every selected block m
// of the ascending list (additive log gate, one scalar per 64x64 tile); an
// online softmax (running max / sum, rescaled accumulator) never materialises
// the attention matrix; O = acc / l and LSE = m + log l.
//
// gfx950 mapping
//  * One workgroup per (batch, kv head, query block, chunk of NW query heads);
//    each wavefront owns the 64 query rows of one head, so the G heads of a
//    kv group share every K/V tile staged in LDS (GQA reuse through LDS).
//  * The scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: in the accumulator layout a lane then holds
//    one query column and 4 consecutive keys of each 16-key tile, so
//      - the row max needs only two cross-lane steps (permlane16/32 swaps),
//      - the row sum stays per lane until the end,
//      - the probabilities are already in the B-operand layout of
//        O^T += V^T P^T (keys permuted consistently on both operands), so P
//        never goes through LDS.
//  * K tiles are kept row-major in LDS (A operand of K Q^T: 16-byte reads);
//    V tiles are written transposed ([d][key]) when staged, so the A operand
//    of V^T P^T is two 8-byte reads.  Row strides are padded so the 16 rows
//    read by one lane group fall in distinct banks.
//  * K/V tiles are double buffered: the next tile's global loads are issued
//    before the current tile's matrix work and written to the other LDS
//    stage after it (one barrier per tile).
//  * Workgroup ids are remapped so that each XCD (own L2) works through a
//    contiguous range of (batch, kv head, query block) units.
#include <math.h>

#include "sas_internal.h"

namespace sas {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BLK = 64;
constexpr int HD = 128;
constexpr int KSTR = HD + 8;   // bf16 per row of a row-major [key][d] LDS tile (272 B)
constexpr int TSTR = BLK + 4;  // bf16 per row of a transposed [d][key] LDS tile (136 B)

struct FwdArgs {
  const bf16* q; const bf16* k; const bf16* v;
  const float* lg; const int32_t* sel_idx; const int32_t* sel_cnt;
  void* o; float* lse;
  int Hq, Hkv, G, N, C, cap;
  int o_fp32;     // store o as float32 (else bf16)
  int head_base;  // first head (within its kv group) of chunk 0 of this launch
  int nchunk;     // chunks of NW heads per (batch, kv head, query block)
  float c2;       // sm_scale * log2(e)
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the lanes l, l^16, l^32, l^48 (the four lanes that share a
// query column of a 16x16 accumulator tile)
__device__ __forceinline__ float max4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int NW>
__global__ void __launch_bounds__(NW * 64, 1) fwd_mfma_kernel(FwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KCH = 1024 / NT;  // 16-byte K chunks per thread per tile
  constexpr int VUN = 256 / NT;   // (4 keys x 8 d) V units per thread per tile
  __shared__ __attribute__((aligned(16))) bf16 s_k[2][BLK * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 s_vt[2][HD * TSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int chunk = unit % a.nchunk;
  const int rest = unit / a.nchunk;
  const int i = rest % a.C;
  const int bhk = rest / a.C;
  const int hk = bhk % a.Hkv;
  const int bb = bhk / a.Hkv;
  const int h = hk * a.G + a.head_base + chunk * NW + w;
  const long long row = (long long)bhk * a.C + i;
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  const float* lgrow = a.lg + row * a.C;
  const bf16* kbase = a.k + (long long)bhk * a.N * HD;
  const bf16* vbase = a.v + (long long)bhk * a.N * HD;
  const long long q0 = ((long long)bb * a.Hq + h) * a.N + (long long)i * BLK;

  // Q^T as the B operand of S^T = K Q^T: lane holds query qt*16 + l16 and
  // head dims ks*32 + g4*8 .. +7.  Pre-scaled by nothing (scale is applied to S).
  bf16x8 qf[4][4];
  {
    const bf16* qp = a.q + q0 * HD;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qf[qt][ks] = *(const bf16x8*)(qp + (qt * 16 + l16) * HD + ks * 32 + g4 * 8);
  }

  u32x4 kreg[KCH];
  u32x4 vreg[VUN][4];
  auto gload = [&](int kb) {
    const bf16* kt = kbase + (long long)kb * BLK * HD;
    const bf16* vt = vbase + (long long)kb * BLK * HD;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + r * NT;
      kreg[r] = *(const u32x4*)(kt + (c >> 4) * HD + (c & 15) * 8);
    }
#pragma unroll
    for (int r = 0; r < VUN; ++r) {
      const int u = tid + r * NT;
      const int kg = u >> 4, dg = u & 15;
#pragma unroll
      for (int x = 0; x < 4; ++x) vreg[r][x] = *(const u32x4*)(vt + (kg * 4 + x) * HD + dg * 8);
    }
  };
  auto lstore = [&](int stg) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + r * NT;
      *(u32x4*)(&s_k[stg][(c >> 4) * KSTR + (c & 15) * 8]) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < VUN; ++r) {
      const int u = tid + r * NT;
      const int kg = u >> 4, dg = u & 15;
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const uint32_t w0 = vreg[r][0][z], w1 = vreg[r][1][z];
        const uint32_t w2 = vreg[r][2][z], w3 = vreg[r][3][z];
        u32x2 lo, hi;
        lo[0] = (w0 & 0xffffu) | (w1 << 16);
        lo[1] = (w2 & 0xffffu) | (w3 << 16);
        hi[0] = (w0 >> 16) | (w1 & 0xffff0000u);
        hi[1] = (w2 >> 16) | (w3 & 0xffff0000u);
        *(u32x2*)(&s_vt[stg][(dg * 8 + 2 * z) * TSTR + kg * 4]) = lo;
        *(u32x2*)(&s_vt[stg][(dg * 8 + 2 * z + 1) * TSTR + kg * 4]) = hi;
      }
    }
  };

  f32x4 oacc[8][4];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) oacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[4], lrow[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) { mrow[qt] = -INFINITY; lrow[qt] = 0.0f; }

  const int ntiles = cnt + 1;
  gload(i);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stg = t & 1;
    const bool diag = (t == 0);
    const int kb = diag ? i : sel[t - 1];
    const float beta = diag ? 0.0f : lgrow[kb] * kLog2e;
    if (t + 1 < ntiles) gload(sel[t]);

    const bf16* Ks = s_k[stg];
    const bf16* Vt = s_vt[stg];

    // ---- S^T = K Q^T ----
    f32x4 sacc[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) sacc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 ka = *(const bf16x8*)(Ks + (kt * 16 + l16) * KSTR + ks * 32 + g4 * 8);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) sacc[kt][qt] = mfma16(ka, qf[qt][ks], sacc[kt][qt]);
      }
    }

    // ---- online softmax (base 2) ----
    bf16x8 pb[2][4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int qi = qt * 16 + l16;  // query index inside the block
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float val = sacc[kt][qt][j] * a.c2 + beta;
          if (diag && (kt * 16 + g4 * 4 + j) > qi) val = -INFINITY;
          x[kt * 4 + j] = val;
          mx = fmaxf(mx, val);
        }
      mx = max4(mx);
      const float mnew = fmaxf(mrow[qt], mx);
      const float alpha = exp2f(mrow[qt] - mnew);
      mrow[qt] = mnew;
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[e] = exp2f(x[e] - mnew);
        ps += x[e];
      }
      lrow[qt] = lrow[qt] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[dt][qt] *= alpha;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[k2][qt][e] = (bf16)x[k2 * 8 + e];
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16* vp = Vt + (dt * 16 + l16) * TSTR + k2 * 32 + g4 * 4;
        const bf16x4 lo = *(const bf16x4*)(vp);
        const bf16x4 hi = *(const bf16x4*)(vp + 16);
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) oacc[dt][qt] = mfma16(va, pb[k2][qt], oacc[dt][qt]);
      }
    }

    if (t + 1 < ntiles) lstore(stg ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const float ltot = sum4(lrow[qt]);
    const float inv = 1.0f / ltot;
    const long long qrow = q0 + qt * 16 + l16;
    if (g4 == 0) a.lse[qrow] = (mrow[qt] + log2f(ltot)) * kLn2;
    if (a.o_fp32) {
      float* op = (float*)a.o + qrow * HD + g4 * 4;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *(f32x4*)(op + dt * 16) = oacc[dt][qt] * inv;
    } else {
      bf16* op = (bf16*)a.o + qrow * HD + g4 * 4;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        bf16x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (bf16)(oacc[dt][qt][j] * inv);
        *(bf16x4*)(op + dt * 16) = r;
      }
    }
  }
}

template <int NW>
hipError_t launch_chunks(FwdArgs a, int head_base, int nchunk, long long units,
                         hipStream_t st) {
  a.head_base = head_base;
  a.nchunk = nchunk;
  const long long grid = units * nchunk;
  hipLaunchKernelGGL((fwd_mfma_kernel<NW>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const Shape& s, const void* q, const void* k, const void* v,
                           const float* log_gate, const int32_t* sel_idx, const int32_t* sel_cnt,
                           void* o, float* lse, hipStream_t st) {
  FwdArgs a{};
  a.q = (const bf16*)q; a.k = (const bf16*)k; a.v = (const bf16*)v;
  a.lg = log_gate; a.sel_idx = sel_idx; a.sel_cnt = sel_cnt;
  a.o = o; a.lse = lse;
  a.o_fp32 = s.o_fp32;
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G; a.N = s.N; a.C = s.C; a.cap = s.cap;
  a.c2 = s.scale * kLog2e;
  const long long units = (long long)s.B * s.Hkv * s.C;
  // the G heads of a group are covered by chunks of 4, then 2, then 1 heads
  int h = 0;
  hipError_t e = hipSuccess;
  if (s.G / 4 > 0) {
    e = launch_chunks<4>(a, h, s.G / 4, units, st);
    h += 4 * (s.G / 4);
    if (e != hipSuccess) return e;
  }
  if ((s.G - h) / 2 > 0) {
    e = launch_chunks<2>(a, h, (s.G - h) / 2, units, st);
    h += 2 * ((s.G - h) / 2);
    if (e != hipSuccess) return e;
  }
  if (s.G - h > 0) e = launch_chunks<1>(a, h, s.G - h, units, st);
  return e;
}

}  // namespace sas
