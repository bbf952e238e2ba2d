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
//  * One workgroup per (batch, kv head, query block, chunk of query heads
//    (2, or 1 for an odd remainder)); two wavefronts per head, each owning
//    32 of its 64 query rows, so the heads of a chunk share every K/V tile
//    staged in LDS, two wavefronts share each SIMD and two workgroups each
//    CU.
//  * The scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: in the accumulator layout a lane then holds
//    one query column and 16 keys of each 32-key half tile, so
//      - the row max needs one cross-lane step (a permlane32 swap),
//      - the row sum stays per lane until the end,
//      - the probabilities, packed pairwise to bf16, are already the B
//        operand of O^T += V^T P^T (keys permuted consistently on both
//        operands), so P never goes through LDS.
//  * K and V tiles are copied global -> LDS asynchronously (global_load_lds,
//    no registers), row-major with an XOR-swizzled 16-byte chunk order.  The
//    A operand of K Q^T is one 16-byte read; the A operand of V^T P^T (a
//    column fragment of V) comes from two transposed reads
//    (ds_read_b64_tr_b16), so V is never transposed in memory.
//  * Two LDS stages per tensor, software-pipelined over half tiles (one
//    barrier per half tile); the tile loop is unrolled by two so each
//    window's stage is a compile-time constant.
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BLK = 64;
constexpr int HD = 128;
constexpr int TILE = BLK * HD;  // bf16 elements of one 64 x 128 K or V tile (16 KB)

struct FwdArgs {
  const bf16* q; const bf16* k; const bf16* v;
  const float* lg; const int32_t* sel_idx; const int32_t* sel_cnt;
  void* o; float* lse;
  int Hq, Hkv, G, N, C, cap;
  int Hs, Gs;     // score heads (gate-table rows per batch) and query heads per score head
  int hard;       // hard Top-K gates: the selected blocks carry unit gates
  int outer;      // outer gate position
  int o_fp32;     // store o as float32 (else bf16)
  int head_base;  // first head (within its kv group) of chunk 0 of this launch
  int nchunk;     // chunks of NW heads per (batch, kv head, query block)
  float c2;       // sm_scale * log2(e)
  const int32_t* lens;   // variable-length batch: valid tokens per sequence (or nullptr)
  const int32_t* cu;     // packed batch: token offsets [B + 1] (or nullptr)
  long long T;           // packed batch: total tokens
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_bf16.  Lane l (g = l / 32): A row l % 32, k = 8 g .. +7;
// B column l % 32, same k; C column l % 32, rows 8 (jj / 4) + 4 g + jj % 4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the lanes l, l^16, l^32, l^48 (the four lanes that share a
// query column of a 16x16 accumulator tile)
__device__ __forceinline__ float max4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// max / sum over the lanes l, l ^ 32 (the two lanes of a 32x32 C column)
__device__ __forceinline__ float max2(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float sum2(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
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
// Row r of the tile is read from g + min(r, rmax) * stride (elements): rows
// are HD apart in the padded layout and Hkv * HD apart in a packed batch,
// whose last rows past a sequence's end repeat its last row (they are
// causally masked; the clamp keeps every read inside the tensor).
template <int NW>
__device__ __forceinline__ void tile_to_lds(bf16* lds, const bf16* g, long long stride, int rmax,
                                            int w, int lane) {
#pragma unroll
  for (int r = 0; r < 16 / NW; ++r) {
    const int seg = w + NW * r;               // 1 KB segment = rows 4 seg .. 4 seg + 3
    const int row = seg * 4 + (lane >> 4);
    const int c = (lane & 15) ^ slot16(row);
    dma16(g + min(row, rmax) * stride + c * 8, lds_addr(lds + seg * 512));
  }
}

__device__ __forceinline__ void wait_vm() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Keeps the computation of x at this point of the instruction stream (the
// vector-ALU work meant to overlap a matrix instruction would otherwise be
// sunk to its first use).
template <typename T>
__device__ __forceinline__ void pin(T& x) { __asm__ volatile("" : "+v"(x)); }

// max(a, b, c) in one v_max3_f32, without the NaN canonicalisation that
// fmaxf gets in IEEE mode (for values produced by MFMAs and exp2, which are
// never signalling NaNs)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Rescale threshold of the lazy online softmax (log2 units): the running max
// is only moved (and O, l rescaled) when a tile raises some row's max by more
// than this; otherwise exp2 arguments stay <= kLazy, so P <= 2^kLazy.
constexpr float kLazy = 8.0f;
// Floor of the running max of a key-split wavefront (log2 units): far below
// any score, far above -inf, so exp2(x - floor) of a masked key stays 0.
constexpr float kMaskFloor = 1.0e30f;

// One workgroup = NH query heads of one (batch, kv head, query block); two
// wavefronts per head, each owning 32 of the 64 query rows (two 16-row tiles).
// At <= 256 registers per wavefront two wavefronts share a SIMD.
// SPLIT: P enters O^T += V^T P^T as hi + lo bf16 terms (two MFMAs), which
// makes O accurate to ~2^-16 relative instead of ~2^-9 (used when o is kept
// in fp32, so the backward's Delta = rowsum(O dO) is exact to fp32 level).
//
// Software pipeline over half tiles: unit u = 2t + kh is keys kh*32 .. +31 of
// tile t (t = 0: the diagonal block, t = 1 .. cnt: the selected blocks).
// Window u holds S_{u+1} = K Q^T (matrix core) interleaved with the softmax
// of S_u (vector ALU), then O^T += V_u^T P_u, and ends with a barrier.
// K and V tiles live in two LDS slots each; window (t, 0) copies V_{t+1} and
// window (t, 1) copies K_{t+2} (their slots' previous tiles were last read in
// window (t - 1, 1) and (t, 0)), and each window waits only for the copies of
// the window before it.
template <int NW>
__device__ __forceinline__ void wait_vm_prev() {   // all but this window's 16 / NW copies
  if (NW == 8) __asm__ volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if (NW == 4) __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory");
}

// OUTER: the outer gate position (Sec. 4.1, Tab. 1 row 3): no logit bias;
// the probabilities of a tile enter O += P V scaled by the tile's gate, while
// the normaliser l sums the unscaled ones.
//
// KS (one head, four wavefronts): the keys of every tile are split between
// two wavefront pairs, wavefront (kq, half) taking keys kq*32 .. +31 for its
// 32 query rows.  One window per tile: S of the wave's next unit (tile t + 1)
// with the softmax of unit t, then its PV; window t copies V_{t+1} and
// K_{t+2} into the slots window t - 1 released.  The two key halves' running
// max, sum and O meet in LDS at the end (the usual softmax merge).  This
// gives a one-head workgroup (per-head gates) four wavefronts on the same
// 64 KB of K / V slots, so two such workgroups fill a CU's SIMDs twice.
template <int NH, bool SPLIT, bool PACKED, bool OUTER, bool KS = false>
__global__ void __launch_bounds__(NH * 128 * (KS ? 2 : 1), 2) fwd_mfma_kernel(FwdArgs a) {
  static_assert(!KS || NH == 1, "the key split is for one-head workgroups");
  constexpr int NW = 2 * NH * (KS ? 2 : 1);
  __shared__ __attribute__((aligned(16))) bf16 s_k[2][TILE];
  __shared__ __attribute__((aligned(16))) bf16 s_v[2][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;          // half of the 32x32 operand k range
  const int l32 = lane & 31;        // query column of this lane
  const int half = w & 1;           // rows half*32 .. half*32 + 31 of the block
  const int kq = KS ? (w >> 1) : 0;   // KS: this wave's key half of every tile

  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int chunk = unit % a.nchunk;
  const int rest = unit / a.nchunk;
  const int i = rest % a.C;
  const int bhk = rest / a.C;
  const int hk = bhk % a.Hkv;
  const int bb = bhk / a.Hkv;
  const int h = hk * a.G + a.head_base + chunk * NH + (KS ? 0 : (w >> 1));
  // gate-table row of this workgroup's heads (all of a chunk share it: with
  // per-head gates a chunk is one head)
  const long long row = ((long long)bb * a.Hs + h / a.Gs) * a.C + i;
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  const float* lgrow = a.lg + row * a.C;
  const long long q0 = ((long long)bb * a.Hq + h) * a.N + (long long)i * BLK + half * 32;

  // Variable-length batch: rows past the sequence's length are padding.  In
  // the padded layout they get o = 0 and lse = 0; in a packed batch they do
  // not exist (reads are clamped to the sequence's last row, nothing is
  // written).  A block without a valid row does nothing else.  (Padding rows
  // hold finite values; only valid rows are mixed into a valid row's result:
  // later keys are masked.)
  constexpr bool packed = PACKED;   // packed variable-length batch (compile-time)
  long long start = 0;   // packed: first token of the sequence
  int nb = a.lens == nullptr ? a.N : min(max(a.lens[bb], 0), a.N);
  if (packed) {
    const long long s0 = min(max((long long)a.cu[bb], 0LL), a.T);
    const long long s1 = min(max((long long)a.cu[bb + 1], s0), a.T);
    start = s0;
    nb = (int)min(s1 - s0, (long long)a.N);
  }
  // K / V rows: tile kb starts at kv_tile(kb); consecutive tokens kv_stride apart
  const long long kv_stride = packed ? (long long)a.Hkv * HD : HD;
  auto kv_tile = [&](int kb) -> long long {
    return packed ? ((start + (long long)kb * BLK) * a.Hkv + hk) * HD
                  : ((long long)bhk * a.N + (long long)kb * BLK) * HD;
  };
  auto kv_rmax = [&](int kb) { return packed ? min(BLK - 1, nb - 1 - kb * BLK) : BLK - 1; };
  if (i * BLK >= nb) {   // uniform over the workgroup: no copy or barrier has been issued
    if (packed || kq != 0) return;
    const long long qrow = q0 + l32;
    if (g == 0) a.lse[qrow] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        if (a.o_fp32)
          *(f32x4*)((float*)a.o + qrow * HD + g * 4 + dt * 32 + q4 * 8) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        else
          *(bf16x4*)((bf16*)a.o + qrow * HD + g * 4 + dt * 32 + q4 * 8) =
              bf16x4{(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
      }
    return;
  }
  const bool row_valid = i * BLK + half * 32 + l32 < nb;
  // this lane's query row (q and o): padded index, or the packed token
  // (clamped to the sequence's last row)
  const int tok = min(i * BLK + half * 32 + l32, nb - 1);
  const long long qrow_i = packed ? (start + tok) * a.Hq + h : q0 + l32;
  const long long lse_i = packed ? (long long)h * a.T + start + tok : q0 + l32;

  // Q^T as the B operand of S^T = K Q^T (32x32x16): lane holds query row
  // l32 and head dims ks*16 + g*8 .. +7 (loaded in the prologue below)
  bf16x8 qf[8];

  // The row's selection, 64 entries at a time, in registers: lane e holds
  // block sel[e0 + e] and its log gate (log2 units); read with readlane.
  int selv = 0;
  float betav = 0.0f;
  int selwin = 0;   // e0 / 64 of the entries in selv
  auto load_sel = [&](int e0) {
    const int e = e0 + lane;
    selv = e < cnt ? sel[e] : 0;
    betav = (e < cnt && !a.hard) ? lgrow[selv] * kLog2e : 0.0f;   // hard gates: unit
    // both loads complete inside this (rarely taken) branch: a load still in
    // flight at the join would make the compiler wait for every outstanding
    // memory operation there, i.e. for the tile copies of the previous window
    // at the start of every window
    settle(selv);
    settle(betav);
  };
  // block and log gate of tile t (t = 0: the diagonal block, gate 0; tiles
  // past the end: the diagonal block again); asked for in increasing order
  const int nt = cnt + 1;
  auto tile_block = [&](int t, float& beta) -> int {
    if (t == 0 || t >= nt) { beta = 0.0f; return i; }
    const int e = t - 1;
    if ((e >> 6) != selwin) { selwin = e >> 6; load_sel(selwin * 64); }
    beta = lane_value(betav, e & 63);
    return lane_value(selv, e & 63);
  };

  // O^T (lane: head dims dt*32 + 8 (jj/4) + 4 g + jj%4, query l32)
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int x = 0; x < 16; ++x) oacc[dt][x] = 0.0f;
  float mrow, lrow = 0.0f;   // running max (log2 units), per-lane partial sum

  // S^T of keys kh*32 .. +31 of the K tile in Ks (lane: query l32, keys
  // 8 (jj/4) + 4 g + jj%4); after MFMA m (m = 0..7) the work per_mfma(m) is
  // issued (sched_barrier keeps the interleave)
  // (the K fragments are read by load_ka, issued before a window's V^T
  // reads so that the first product does not queue behind them)
  auto load_ka = [&](const bf16* Ks, int kh, bf16x8 (&ka)[8]) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ka[ks] = *(const bf16x8*)(Ks + swz(kh * 32 + l32, ks * 2 + g));
  };
  auto scores_from = [&](const bf16x8 (&ka)[8], f32x16& sc, auto&& per_mfma) {
#pragma unroll
    for (int x = 0; x < 16; ++x) sc[x] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sc = mfma32(ka[ks], qf[ks], sc);
      per_mfma(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto scores_with = [&](const bf16* Ks, int kh, f32x16& sc, auto&& per_mfma) {
    bf16x8 ka[8];
    load_ka(Ks, kh, ka);
    scores_from(ka, sc, per_mfma);
  };
  // causal mask of the diagonal tile: key > query -> -inf
  auto mask_diag = [&](int kh, f32x16& sc) {
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      if (kh * 32 + (jj >> 2) * 8 + g * 4 + (jj & 3) > half * 32 + l32) sc[jj] = -INFINITY;
  };
  // running max over a unit's keys (FIRST: the max starts here; otherwise O
  // and l are rescaled only when the row's max grows by more than kLazy)
  auto update_max = [&](auto first_tag, const f32x16& sc, float beta) {
    constexpr bool FIRST = decltype(first_tag)::value;
    // v_max3 chains; the row's other 16 keys sit in lane l ^ 32
    float mx = max3f(sc[0], sc[1], sc[2]);
#pragma unroll
    for (int jj = 3; jj < 15; jj += 2) mx = max3f(mx, sc[jj], sc[jj + 1]);
    mx = max3f(mx, sc[15], sc[15]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                     false, false);
    mx = max3f(mx, __uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float tmax = mx * a.c2 + beta;
    if (FIRST) {
      // KS: a wave's first unit can be wholly masked (keys 32..63 of the
      // diagonal tile for rows 0..31): a finite floor keeps exp2 at 0 there
      mrow = KS ? fmaxf(tmax, -kMaskFloor) : tmax;
    } else if (__builtin_amdgcn_ballot_w64(tmax > mrow + kLazy) != 0) {   // wave-uniform, rare
      const float mnew = fmaxf(mrow, tmax);
      const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
      mrow = mnew;
      lrow *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
    }
  };
  // P element pair n (n = 0..7) of a unit: P = exp2(c2 s + beta - m), summed
  // into l and packed (hi, and lo when SPLIT) into the B operand of
  // O^T += V^T P^T: element jj -> k-slice jj / 8, word (jj % 8) / 2
  auto p_pair = [&](int n, const f32x16& sc, float off, float gv, uint32_t (&pb)[2][4],
                    uint32_t (&pl)[2][4]) {
    const int jj = 2 * n;
    const f32x2 p0 = {__builtin_amdgcn_exp2f(fmaf(sc[jj], a.c2, off)),
                      __builtin_amdgcn_exp2f(fmaf(sc[jj + 1], a.c2, off))};
    const f32x2 pp = OUTER ? f32x2{p0[0] * gv, p0[1] * gv} : p0;   // outer: g P enters O
    const bf16x2 hi = __builtin_convertvector(pp, bf16x2);
    uint32_t wh = __builtin_bit_cast(uint32_t, hi);
    pin(wh);
    pb[jj >> 3][(jj & 7) >> 1] = wh;
    if (OUTER || SPLIT) {
      lrow += p0[0] + p0[1];   // the unscaled (outer) or unrounded (split) weights
    } else {
      // the bf16 weights that enter O, one dot product per pair
      lrow = __builtin_amdgcn_fdot2_f32_bf16(hi, bf16x2{(bf16)1.0f, (bf16)1.0f}, lrow, false);
    }
    if (SPLIT) {
      const bf16x2 lo = __builtin_convertvector(pp - __builtin_convertvector(hi, f32x2), bf16x2);
      uint32_t wl = __builtin_bit_cast(uint32_t, lo);
      pin(wl);
      pl[jj >> 3][(jj & 7) >> 1] = wl;
    }
  };
  // O^T += V^T P^T over keys kh*32 .. +31.  V^T fragments (A operand, lane:
  // head dim dt*32 + l32, keys 16 sl + {4g .. 4g+3, 8+4g .. 8+4g+3}) come from
  // transposed reads of the row-major V tile.
  const int u = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  int tro[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      tro[dt][hh] = swz(g * 4 + (u >> 2) + 8 * hh, dt * 4 + dhalf * 2 + ((u >> 1) & 1)) + (u & 1) * 4;
  // the V^T fragments of a unit are read at the start of its window, so their
  // LDS latency hides behind the S products and the softmax of the window
  auto read_va = [&](const bf16* Vs, int kh, bf16x8 (&va)[4][2]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const bf16* vp = Vs + (kh * 32 + sl * 16) * HD;
        va[dt][sl] = __builtin_shufflevector(ds_read_tr(vp + tro[dt][0]), ds_read_tr(vp + tro[dt][1]),
                                             0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  auto pv = [&](const bf16x8 (&va)[4][2], const uint32_t (&pbw)[2][4], const uint32_t (&plw)[2][4]) {
    bf16x8 pb[2], pl[2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      pb[sl] = __builtin_bit_cast(bf16x8, u32x4{pbw[sl][0], pbw[sl][1], pbw[sl][2], pbw[sl][3]});
      pl[sl] = __builtin_bit_cast(bf16x8, u32x4{plw[sl][0], plw[sl][1], plw[sl][2], plw[sl][3]});
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        oacc[dt] = mfma32(va[dt][sl], pb[sl], oacc[dt]);
        if (SPLIT) oacc[dt] = mfma32(va[dt][sl], pl[sl], oacc[dt]);
      }
  };

  // this lane's byte offsets in a tile for the wave's 1 KB segments (rows
  // 4 seg .. 4 seg + 3, seg = w + NW r), swizzled as tile_to_lds does; the
  // padded layout copies with one scalar base per tile
  unsigned voff[16 / NW];
#pragma unroll
  for (int r = 0; r < 16 / NW; ++r) {
    const int rr = (w + NW * r) * 4 + (lane >> 4);
    voff[r] = (unsigned)(rr * HD + (((lane & 15) ^ slot16(rr)) << 3)) * 2;
  }
  auto copy_tile = [&](const bf16* src, bf16* lds, int kb) {
    if (packed) {   // rows clamped per lane to the sequence's last row
      tile_to_lds<NW>(lds, src + kv_tile(kb), kv_stride, kv_rmax(kb), w, lane);
    } else {
      const bf16* base = src + kv_tile(kb);
#pragma unroll
      for (int r = 0; r < 16 / NW; ++r) dma16s(base, voff[r], lds_addr(lds + (w + NW * r) * 512));
    }
  };
  auto copy_k = [&](int kb, int slot) { copy_tile(a.k, s_k[slot], kb); };
  auto copy_v = [&](int kb, int slot) { copy_tile(a.v, s_v[slot], kb); };

  // prologue: K_0, V_0, K_1 in; S of unit 0 (masked) starts the running max.
  // The diagonal tiles' copies, the Q rows and the selection (read up to the
  // capacity, so without waiting for the count) go out together; then K of
  // tile 1 and the gate gather, which need the selection: two memory
  // latencies instead of the four of count, selection, gates, copies.
  float beta1 = 0.0f;
  copy_k(i, 0);
  copy_v(i, 0);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = *(const bf16x8*)(a.q + qrow_i * HD + ks * 16 + g * 8);
  {
    const int raw = lane < a.cap ? sel[lane] : 0;
    selv = lane < cnt ? raw : 0;
  }
  copy_k(nt > 1 ? lane_value(selv, 0) : i, 1);
  betav = (lane < cnt && !a.hard) ? lgrow[selv] * kLog2e : 0.0f;
  settle(betav);
  if (nt > 1) beta1 = lane_value(betav, 0);
  wait_vm();
  __syncthreads();
  f32x16 s0, s1;   // S of the unit being finished / the next unit
  scores_with(s_k[0], kq, s0, [](int) {});
  mask_diag(kq, s0);
  update_max(std::true_type{}, s0, 0.0f);

  // window (t, kh): copy (V_{t+1} for kh = 0, K_{t+2} for kh = 1); S of the
  // next unit with the softmax of this one; O += V^T P; barrier; max of the
  // next unit
  float beta_cur = 0.0f;   // gate of tile t
  float beta_v = beta1;    // gate of the tile whose V was copied last (t + 1)
  // PAR = t & 1 (a compile-time LDS slot, so the fragment addresses are
  // loop invariant)
  auto window = [&](auto kh_tag, auto diag_tag, auto par_tag, int t, f32x16& scur, f32x16& snext) {
    constexpr int KH = decltype(kh_tag)::value;
    constexpr bool DIAG = decltype(diag_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    const bool more = KH == 0 || t + 1 < nt;   // is there a next unit
    if (KH == 0) {
      copy_v(tile_block(t + 1, beta_v), PAR ^ 1);
    } else {
      float bk;
      copy_k(tile_block(t + 2, bk), PAR);
    }
    const float off = (OUTER ? 0.0f : beta_cur) - mrow;
    const float gvw = OUTER ? __builtin_amdgcn_exp2f(beta_cur) : 1.0f;   // outer: the tile's gate
    uint32_t pb[2][4], pl[2][4];
    bf16x8 va[4][2];
    // next unit: (t, 1) reads K_t, (t + 1, 0) reads K_{t+1}
    const bf16* kn = KH == 0 ? s_k[PAR] : s_k[PAR ^ 1];
    // K fragments first (not with split P, whose lo terms leave no
    // registers for both sets in flight)
    constexpr bool K_FIRST = !SPLIT;
    bf16x8 ka[8];
    if (K_FIRST && more) load_ka(kn, KH ^ 1, ka);
    // (a packed batch's per-lane clamped copies leave no registers for the
    // early read: there the fragments are read just before the product)
    if (!PACKED) read_va(s_v[PAR], KH, va);
    if (more) {
      if (!K_FIRST) load_ka(kn, KH ^ 1, ka);
      scores_from(ka, snext, [&](int m) { p_pair(m, scur, off, gvw, pb, pl); });
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) p_pair(n, scur, off, gvw, pb, pl);
    }
    if (PACKED) read_va(s_v[PAR], KH, va);
    pv(va, pb, pl);
    wait_vm_prev<NW>();
    __syncthreads();
    if (more) {
      if (KH == 0) {
        if (DIAG) mask_diag(1, snext);
        update_max(std::false_type{}, snext, OUTER ? 0.0f : beta_cur);
      } else {
        beta_cur = beta_v;   // tile t + 1
        update_max(std::false_type{}, snext, OUTER ? 0.0f : beta_cur);
      }
    }
  };
  // KS window t (PAR = t & 1): V_{t+1} -> V slot PAR ^ 1 and K_{t+2} -> K
  // slot PAR (both last read in window t - 1); S of unit (t + 1, kq) from K
  // slot PAR ^ 1 with the softmax of unit (t, kq); O += V_t^T P; the copies
  // land before the barrier (window t + 1 reads both)
  auto window_ks = [&](auto par_tag, int t, f32x16& scur, f32x16& snext) {
    constexpr int PAR = decltype(par_tag)::value;
    const bool more = t + 1 < nt;
    copy_v(tile_block(t + 1, beta_v), PAR ^ 1);
    {
      float bk;
      copy_k(tile_block(t + 2, bk), PAR);
    }
    const float off = (OUTER ? 0.0f : beta_cur) - mrow;
    const float gvw = OUTER ? __builtin_amdgcn_exp2f(beta_cur) : 1.0f;
    uint32_t pb[2][4], pl[2][4];
    bf16x8 va[4][2];
    if (!PACKED) read_va(s_v[PAR], kq, va);
    if (more) {
      scores_with(s_k[PAR ^ 1], kq, snext, [&](int m) { p_pair(m, scur, off, gvw, pb, pl); });
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) p_pair(n, scur, off, gvw, pb, pl);
    }
    if (PACKED) read_va(s_v[PAR], kq, va);
    pv(va, pb, pl);
    wait_vm();
    __syncthreads();
    if (more) {
      beta_cur = beta_v;   // tile t + 1
      update_max(std::false_type{}, snext, OUTER ? 0.0f : beta_cur);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (KS) {
    __syncthreads();   // every wave's S of unit 0 has read K slot 0 (window 0 refills it)
    window_ks(I0{}, 0, s0, s1);
    int t = 1;
#pragma unroll 1
    for (; t + 1 < nt; t += 2) {   // tiles t (odd) and t + 1 (even)
      window_ks(I1{}, t, s1, s0);
      window_ks(I0{}, t + 1, s0, s1);
    }
    if (t < nt) window_ks(I1{}, t, s1, s0);
  } else {
    window(I0{}, std::true_type{}, I0{}, 0, s0, s1);
    window(I1{}, std::true_type{}, I0{}, 0, s1, s0);
    int t = 1;
#pragma unroll 1
    for (; t + 1 < nt; t += 2) {   // tiles t (odd) and t + 1 (even)
      window(I0{}, std::false_type{}, I1{}, t, s0, s1);
      window(I1{}, std::false_type{}, I1{}, t, s1, s0);
      window(I0{}, std::false_type{}, I0{}, t + 1, s0, s1);
      window(I1{}, std::false_type{}, I0{}, t + 1, s1, s0);
    }
    if (t < nt) {
      window(I0{}, std::false_type{}, I1{}, t, s0, s1);
      window(I1{}, std::false_type{}, I1{}, t, s1, s0);
    }
  }
  wait_vm();   // trailing copies

  if (KS) {
    // merge the key halves: the kq = 1 waves leave m, their partial sums and
    // O^T in LDS (K slots: O, lane-major 16-byte vectors; V slot 0: m, l),
    // the kq = 0 waves fold them into their own and write the rows
    __syncthreads();   // every wave is done with the K / V slots
    f32x4* xo = (f32x4*)&s_k[0][0] + half * 16 * 64 + lane;
    float* xm = (float*)&s_v[0][0] + (half * 64 + lane) * 2;
    if (kq == 1) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xo[(dt * 4 + q4) * 64] = f32x4{oacc[dt][q4 * 4], oacc[dt][q4 * 4 + 1], oacc[dt][q4 * 4 + 2],
                                         oacc[dt][q4 * 4 + 3]};
      xm[0] = mrow;
      xm[1] = lrow;
    }
    __syncthreads();
    if (kq == 1) return;
    const float mb = xm[0];
    const float mnew = fmaxf(mrow, mb);
    const float aa = __builtin_amdgcn_exp2f(mrow - mnew);
    const float ab = __builtin_amdgcn_exp2f(mb - mnew);
    lrow = lrow * aa + xm[1] * ab;
    mrow = mnew;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 ob = xo[(dt * 4 + q4) * 64];
#pragma unroll
        for (int y = 0; y < 4; ++y) oacc[dt][q4 * 4 + y] = oacc[dt][q4 * 4 + y] * aa + ob[y] * ab;
      }
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----
  const float ltot = sum2(lrow);
  const float inv = row_valid ? 1.0f / ltot : 0.0f;   // padding rows: o = 0, lse = 0
  if (packed && !row_valid) return;   // the row belongs to no sequence of this batch
  const long long qrow = qrow_i;
  if (g == 0) a.lse[lse_i] = row_valid ? (mrow + log2f(ltot)) * kLn2 : 0.0f;
  if (a.o_fp32) {
    float* op = (float*)a.o + qrow * HD + g * 4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4*)(op + dt * 32 + q4 * 8) =
            f32x4{oacc[dt][q4 * 4] * inv, oacc[dt][q4 * 4 + 1] * inv, oacc[dt][q4 * 4 + 2] * inv,
                  oacc[dt][q4 * 4 + 3] * inv};
  } else {
    bf16* op = (bf16*)a.o + qrow * HD + g * 4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 r;
#pragma unroll
        for (int y = 0; y < 4; ++y) r[y] = (bf16)(oacc[dt][q4 * 4 + y] * inv);
        *(bf16x4*)(op + dt * 32 + q4 * 8) = r;
      }
  }
}

template <int NH, bool KS = false>
hipError_t launch_chunks(FwdArgs a, int head_base, int nchunk, long long units,
                         hipStream_t st) {
  a.head_base = head_base;
  a.nchunk = nchunk;
  const dim3 grid((unsigned)(units * nchunk)), block(NH * 128 * (KS ? 2 : 1));
  const int v = (a.o_fp32 ? 4 : 0) | (a.cu != nullptr ? 2 : 0) | (a.outer ? 1 : 0);
  switch (v) {
    case 0: hipLaunchKernelGGL((fwd_mfma_kernel<NH, false, false, false, KS>), grid, block, 0, st, a); break;
    case 1: hipLaunchKernelGGL((fwd_mfma_kernel<NH, false, false, true, KS>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((fwd_mfma_kernel<NH, false, true, false, KS>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((fwd_mfma_kernel<NH, false, true, true, KS>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((fwd_mfma_kernel<NH, true, false, false, KS>), grid, block, 0, st, a); break;
    case 5: hipLaunchKernelGGL((fwd_mfma_kernel<NH, true, false, true, KS>), grid, block, 0, st, a); break;
    case 6: hipLaunchKernelGGL((fwd_mfma_kernel<NH, true, true, false, KS>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((fwd_mfma_kernel<NH, true, true, true, KS>), grid, block, 0, st, a); break;
  }
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
  a.lens = s.lens;
  a.cu = s.cu;
  a.T = s.T;
  a.Hs = s.Hs;
  a.Gs = s.Hq / s.Hs;
  a.hard = s.hard;
  a.outer = s.outer;
  const long long units = (long long)s.B * s.Hkv * s.C;
  if (a.Gs < 2) {   // gates per query head: every head selects its own blocks
    // (one head per workgroup, its tiles' keys split over two wave pairs)
    return launch_chunks<1, true>(a, 0, s.G, units, st);
  }
  // the G heads of a group are covered by chunks of 2 heads, then 1: two
  // 4-wavefront workgroups per CU drift out of step, so one's barrier and
  // softmax phases overlap the other's matrix work (a chunk of 4 heads in one
  // 8-wavefront workgroup shares each K / V tile more widely but was 2.6 %
  // slower at the 32k shape)
  int h = 0;
  hipError_t e = hipSuccess;
  if ((s.G - h) / 2 > 0) {
    e = launch_chunks<2>(a, h, (s.G - h) / 2, units, st);
    h += 2 * ((s.G - h) / 2);
    if (e != hipSuccess) return e;
  }
  if (s.G - h > 0) e = launch_chunks<1>(a, h, s.G - h, units, st);
  return e;
}

}  // namespace sas
