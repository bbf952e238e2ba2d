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
//  * One workgroup per (batch, kv head, query block, chunk of query heads);
//    two wavefronts per head, each owning 32 of its 64 query rows, so the G
//    heads of a kv group share every K/V tile staged in LDS (GQA reuse
//    through LDS) and two wavefronts share each SIMD.
//  * The scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: in the accumulator layout a lane then holds
//    one query column and 4 consecutive keys of each 16-key tile, so
//      - the row max needs only two cross-lane steps (permlane16/32 swaps),
//      - the row sum stays per lane until the end,
//      - the probabilities are already in the B-operand layout of
//        O^T += V^T P^T (keys permuted consistently on both operands), so P
//        never goes through LDS.
//  * K and V tiles are copied global -> LDS asynchronously (global_load_lds,
//    no registers), row-major with an XOR-swizzled 16-byte chunk order.  The
//    A operand of K Q^T is one 16-byte read; the A operand of V^T P^T (a
//    column fragment of V) comes from two transposed reads
//    (ds_read_b64_tr_b16), so V is never transposed in memory.
//  * Two LDS stages: the next tile's copy is issued before the current
//    tile's matrix work (one barrier per tile).
//  * The online softmax rescales O lazily (only when a row max grows by more
//    than 2^8) and the diagonal tile is peeled, so the steady-state tile has
//    no masking and, almost always, no accumulator rescale.
//  * Workgroup ids are remapped so that each XCD (own L2) works through a
//    contiguous range of (batch, kv head, query block) units.
#include <math.h>

#include <type_traits>

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
constexpr int TILE = BLK * HD;  // bf16 elements of one 64 x 128 K or V tile (16 KB)

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

// gfx950 transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane u receives element u % 4 of the 8-byte chunks addressed by lanes
// u / 4 + 4x (x = 0..3).  With lane u addressing row base + u / 4, columns
// c0 + 4 (u % 4) .. +3 of a row-major tile, lane u gets rows base .. base + 3
// of column c0 + u.
__device__ __forceinline__ bf16x4 ds_read_tr(const bf16* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// LDS tiles are row-major with 256-byte rows and no padding; the 16-byte chunk
// c of row r sits in slot c ^ (r & 15).  The 16 rows read by one lane group
// (same chunk) then fall in 16 different slots, i.e. all 64 banks.
__device__ __forceinline__ int swz(int r, int c) { return r * HD + ((c ^ slot16(r)) << 3); }

// Asynchronous global -> LDS copy of one 64 x 128 tile by NW wavefronts
// (global_load_lds_dwordx4: each instruction writes 64 x 16 contiguous bytes
// of LDS; the lanes pick their global chunk so the result is swizzled).
// Completion is waited for with s_waitcnt vmcnt(0) before the next barrier.
template <int NW>
__device__ __forceinline__ void tile_to_lds(bf16* lds, const bf16* g, int w, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int r = 0; r < 16 / NW; ++r) {
    const int seg = w + NW * r;               // 1 KB segment = rows 4 seg .. 4 seg + 3
    const int row = seg * 4 + (lane >> 4);
    const int c = (lane & 15) ^ slot16(row);
    dma16(g + row * HD + c * 8, lds_addr(lds + seg * 512));
  }
}

__device__ __forceinline__ void wait_vm() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Rescale threshold of the lazy online softmax (log2 units): the running max
// is only moved (and O, l rescaled) when a tile raises some row's max by more
// than this; otherwise exp2 arguments stay <= kLazy, so P <= 2^kLazy.
constexpr float kLazy = 8.0f;

// One workgroup = NH query heads of one (batch, kv head, query block); two
// wavefronts per head, each owning 32 of the 64 query rows (two 16-row tiles).
// At <= 256 registers per wavefront two wavefronts share a SIMD, so one
// wavefront's softmax runs while the other's matrix instructions issue.
// SPLIT: P enters O^T += V^T P^T as hi + lo bf16 terms (two MFMAs), which
// makes O accurate to ~2^-16 relative instead of ~2^-9 (used when o is kept
// in fp32, so the backward's Delta = rowsum(O dO) is exact to fp32 level).
template <int NH, bool SPLIT>
__global__ void __launch_bounds__(NH * 128, 2) fwd_mfma_kernel(FwdArgs a) {
  constexpr int NW = 2 * NH;
  __shared__ __attribute__((aligned(16))) bf16 s_k[2][TILE];
  __shared__ __attribute__((aligned(16))) bf16 s_v[2][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int half = w & 1;           // rows half*32 .. half*32 + 31 of the block

  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int chunk = unit % a.nchunk;
  const int rest = unit / a.nchunk;
  const int i = rest % a.C;
  const int bhk = rest / a.C;
  const int hk = bhk % a.Hkv;
  const int bb = bhk / a.Hkv;
  const int h = hk * a.G + a.head_base + chunk * NH + (w >> 1);
  const long long row = (long long)bhk * a.C + i;
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  const float* lgrow = a.lg + row * a.C;
  const bf16* kbase = a.k + (long long)bhk * a.N * HD;
  const bf16* vbase = a.v + (long long)bhk * a.N * HD;
  const long long q0 = ((long long)bb * a.Hq + h) * a.N + (long long)i * BLK + half * 32;

  // Q^T as the B operand of S^T = K Q^T: lane holds row qt*16 + l16 (of this
  // wavefront's 32) and head dims ks*32 + g4*8 .. +7.
  bf16x8 qf[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[qt][ks] = *(const bf16x8*)(a.q + (q0 + qt * 16 + l16) * HD + ks * 32 + g4 * 8);

  auto load_tile = [&](int kb, int stg) {
    tile_to_lds<NW>(s_k[stg], kbase + (long long)kb * TILE, w, lane);
    tile_to_lds<NW>(s_v[stg], vbase + (long long)kb * TILE, w, lane);
  };

  f32x4 oacc[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) oacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2], lrow[2];   // running max (log2 units) and per-lane partial sums

  // One 64-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
  auto tile = [&](auto diag_tag, int stg, float beta) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    const bf16* Ks = s_k[stg];
    const bf16* Vs = s_v[stg];
    f32x4 sacc[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) sacc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 ka = *(const bf16x8*)(Ks + swz(kt * 16 + l16, ks * 4 + g4));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) sacc[kt][qt] = mfma16(ka, qf[qt][ks], sacc[kt][qt]);
      }
    }
    if (DIAG) {   // causal mask inside the current block: key > query -> -inf
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (kt * 16 + g4 * 4 + j > half * 32 + qt * 16 + l16) sacc[kt][qt][j] = -INFINITY;
    }
    // tile row max (raw scores; c2 > 0 keeps the order)
    float tmax[2];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = fmaxf(fmaxf(sacc[0][qt][0], sacc[0][qt][1]), fmaxf(sacc[0][qt][2], sacc[0][qt][3]));
#pragma unroll
      for (int kt = 1; kt < 4; ++kt)
        mx = fmaxf(mx, fmaxf(fmaxf(sacc[kt][qt][0], sacc[kt][qt][1]),
                             fmaxf(sacc[kt][qt][2], sacc[kt][qt][3])));
      tmax[qt] = max4(mx) * a.c2 + beta;
      if (!DIAG) grow |= tmax[qt] > mrow[qt] + kLazy;
    }
    if (DIAG) {
      // first tile: O and l are still zero, the max just starts here
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) { mrow[qt] = tmax[qt]; lrow[qt] = 0.0f; }
    } else if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // wave-uniform, rare
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float mnew = fmaxf(mrow[qt], tmax[qt]);
        const float alpha = __builtin_amdgcn_exp2f(mrow[qt] - mnew);
        mrow[qt] = mnew;
        lrow[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt][qt] *= alpha;
      }
    }
    // P = exp2(c2 s + beta - m), packed as the B operand of O^T += V^T P^T
    bf16x8 pb[2][2], pl[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float off = beta - mrow[qt];
      float ps = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][qt][j], a.c2, off));
          ps += p;
          const bf16 ph = (bf16)p;
          pb[kt >> 1][qt][(kt & 1) * 4 + j] = ph;
          if (SPLIT) pl[kt >> 1][qt][(kt & 1) * 4 + j] = (bf16)(p - (float)ph);
        }
      lrow[qt] += ps;
    }
    // O^T += V^T P^T; V^T fragments read transposed from the row-major tile:
    // for head-dim tile dt, rows vr + {0, 16, 32, 48} of column dt*16 + l16
    // (the swizzle slot depends only on the row mod 16, so the four reads are
    // 4 KB apart)
    const int vr = g4 * 4 + (l16 >> 2);
    const unsigned vbase = lds_addr(Vs) + (unsigned)(vr * HD + (l16 & 1) * 4) * 2;
#pragma unroll
    for (int dp = 0; dp < 4; ++dp) {   // two head-dim tiles per batch of reads
      tr_u32x2 r[8];
      tr_read_2x4(vbase + (((dp * 4 + ((l16 >> 1) & 1)) ^ slot16(vr)) << 4),
                  vbase + (((dp * 4 + 2 + ((l16 >> 1) & 1)) ^ slot16(vr)) << 4), r);
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2) {
        const int dt = dp * 2 + d2;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const tr_u32x2 lo = r[d2 * 4 + k2 * 2], hi = r[d2 * 4 + k2 * 2 + 1];
          const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            oacc[dt][qt] = mfma16(va, pb[k2][qt], oacc[dt][qt]);
            if (SPLIT) oacc[dt][qt] = mfma16(va, pl[k2][qt], oacc[dt][qt]);
          }
        }
      }
    }
  };

  // The row's selection, 64 entries at a time, in registers: lane e holds
  // block sel[e0 + e] and its log gate (log2 units); the tile loop reads them
  // with readlane, so it issues no global loads besides the tile copies.
  int selv = 0;
  float betav = 0.0f;
  auto load_sel = [&](int e0) {
    const int e = e0 + lane;
    selv = e < cnt ? sel[e] : 0;
    betav = e < cnt ? lgrow[selv] * kLog2e : 0.0f;
    settle(betav);
  };

  const int ntiles = cnt + 1;
  load_sel(0);
  load_tile(i, 0);
  wait_vm();
  __syncthreads();
  // diagonal tile (unit gate, causal); the next tile streams into the other stage
  float nbeta = 0.0f;   // log gate of the tile in the other stage
  if (ntiles > 1) {
    load_tile(lane_value(selv, 0), 1);
    nbeta = lane_value(betav, 0);
  }
  tile(std::true_type{}, 0, 0.0f);
  wait_vm();
  __syncthreads();
  // selected tiles (additive log gate)
  for (int t = 1; t < ntiles; ++t) {
    const int stg = t & 1;
    const float beta = nbeta;
    if (t + 1 < ntiles) {   // entry t of the selection feeds tile t + 1
      if ((t & 63) == 0) load_sel(t);
      load_tile(lane_value(selv, t & 63), stg ^ 1);
      nbeta = lane_value(betav, t & 63);
    }
    tile(std::false_type{}, stg, beta);
    wait_vm();
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
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

template <int NH>
hipError_t launch_chunks(FwdArgs a, int head_base, int nchunk, long long units,
                         hipStream_t st) {
  a.head_base = head_base;
  a.nchunk = nchunk;
  const long long grid = units * nchunk;
  if (a.o_fp32)
    hipLaunchKernelGGL((fwd_mfma_kernel<NH, true>), dim3((unsigned)grid), dim3(NH * 128), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<NH, false>), dim3((unsigned)grid), dim3(NH * 128), 0, st, a);
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
