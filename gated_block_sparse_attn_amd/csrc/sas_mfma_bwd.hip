// Matrix-core (MFMA) backward of SAS gated block-sparse attention, bf16
// inputs, fp32 accumulation, block b = 64, head_dim D = 128, on gfx950.
//
// Follows the recomputation backward of the SAS paper's App. E (Alg. 4):
//   P = exp(S - LSE);  dS = P * (dO V^T - Delta);
//   dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO;
//   dLogG[i, m] = sum of dS over the query tokens of block i (all G heads of
//                 the kv group) and the key tokens of selected block m;
// and the selector-score gradient of App. D.3 / Eq. 8.  Delta, the row
// correction of App. E, is rowsum(O * dO) = sum_u P_u dP_u.
//
// Kernels (in launch order):
//   bwd_dq_kernel       query-major pass: one workgroup per (batch, kv head,
//                       query block, chunk of heads); each wavefront owns 32
//                       query rows of one head and streams the diagonal block
//                       and the selected blocks.  It recomputes S^T = K Q^T
//                       and dP^T = V dO^T, forms dS with Delta = rowsum(O dO)
//                       and accumulates dQ^T += K^T dS^T in registers; on the
//                       side it sums P * dP of every row (Delta without the
//                       rounding of O), which the key-major pass uses.
//   column kernels      transpose the selection: bit (j, i) of a column mask is
//                       set when row i selected block j; each column j then
//                       gets the ascending list {j} u {i > j : j in I_i} and is
//                       cut into chunks of at most a.cc query blocks,
//                       ordered for L2 reuse.
//   bwd_dkdv_kernel     key-major pass: four wavefronts (two pairs, one per
//                       half of key block j) per column chunk; K_j / V_j are
//                       resident MFMA operands, the (query block, head) rows
//                       stream through LDS rings;
//                       it recomputes S and dP, accumulates dV^T += dO^T P and
//                       dK^T += Q^T dS, and writes dLogG[i, j] of each
//                       selecting query block i (sum of its dS).
//   reduce_kernel       columns cut into several chunks: fp32 partials summed
//                       in chunk order (deterministic).
//   dscores_kernel      (sas_threshold.hip) selector-score gradient from the
//                       dense dLogG table.
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

struct BwdArgs {
  const bf16* q; const bf16* k; const bf16* v; const void* o; const bf16* d_o;
  const float* lse; const float* lg; const int32_t* sel_idx; const int32_t* sel_cnt;
  bf16* dq; bf16* dk; bf16* dv; float* dlg; float* dsc;
  float* delta;
  float* lsen;     // -LSE log2(e) per query row (-inf on padding rows), from the dq pass
  uint32_t* colmask; int32_t* collen; int32_t* coloff; int32_t* chunkoff; int32_t* collist;
  float* partial;
  int32_t* chunk_rank; int32_t* chunk_hist; int32_t* chunk_desc;
  long long nrow;  // B * Hs * C: gate-table rows
  long long ncol;  // B * Hkv * C: key-major columns (batch, kv head, key block)
  int nsh;         // score heads per kv head (Hs / Hkv): a column entry is
                   // (query block i, score head sl of the kv head), code i * nsh + sl
  int Hq, Hkv, G, N, C, cap, W, o_fp32;
  int Hs, Gs;       // score heads (gate-table rows per batch) and query heads per score head
  int hard;         // hard Top-K gates: unit gates on the selected blocks
  int outer;        // outer gate position
  int cc;           // query blocks per key-major chunk
  int head_base, nchunk;
  float c2, scale;
  const int32_t* lens;   // variable-length batch (padded layout): valid tokens, or nullptr
  const int32_t* cu;     // packed batch: token offsets [B + 1], or nullptr
  long long T;           // packed batch: total tokens
};

// First token (packed batch) and valid tokens of sequence b, clamped so that
// every row stays inside the tensors.
struct Span {
  long long start;
  int n;
};
__device__ __forceinline__ Span seq_span(const BwdArgs& a, int b) {
  if (a.cu != nullptr) {
    const long long s0 = min(max((long long)a.cu[b], 0LL), a.T);
    const long long s1 = min(max((long long)a.cu[b + 1], s0), a.T);
    return {s0, (int)min(s1 - s0, (long long)a.N)};
  }
  return {0, a.lens == nullptr ? a.N : min(max(a.lens[b], 0), a.N)};
}

__device__ __forceinline__ float sum2(float x) {   // lanes l, l ^ 32
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// LDS written by some lanes of this wavefront is read by other lanes of the
// same wavefront: wait for the LDS queue and keep the compiler from moving
// memory operations across.
__device__ __forceinline__ void wave_lds_sync() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ bf16x8 join(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// gfx950 transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane u receives element u % 4 of the 8-byte chunks addressed by lanes
// u / 4 + 4x (x = 0..3).  With lane u addressing row base + u / 4, columns
// c0 + 4 (u % 4) .. +3 of a row-major tile, lane u therefore gets rows
// base .. base + 3 of column c0 + u: a column fragment of the tile.
__device__ __forceinline__ bf16x4 ds_read_tr(const bf16* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// ---------------------------------------------------------------------------
// query-major pass: dQ and the row sums of P * dP
// ---------------------------------------------------------------------------
constexpr int TILE = BLK * HD;   // bf16 elements of one 64 x 128 tile

// LDS tiles are row-major with 256-byte rows and no padding; the 16-byte chunk
// c of row r sits in slot c ^ (r & 15), so the 16 rows read by a lane group
// for one chunk land in 16 different slots (all banks).
__device__ __forceinline__ int swz(int r, int c) { return r * HD + ((c ^ slot16(r)) << 3); }

// Asynchronous global -> LDS copy of one 64 x 128 tile by NW wavefronts
// (global_load_lds_dwordx4); completion is awaited with s_waitcnt vmcnt(0).
// Row r comes from g + min(r, rmax) * stride (elements): HD in the padded
// layout, Hkv * HD in a packed batch, where rows past a sequence's end repeat
// its last row (causally masked; the clamp keeps reads inside the tensor).
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

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// v_mfma_f32_32x32x16_bf16.  Lane l (g = l / 32): A row l % 32, k = 8 g .. +7;
// B column l % 32, same k; C column l % 32, rows 8 (jj / 4) + 4 g + jj % 4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One workgroup = NH query heads of one (batch, kv head, query block); two
// wavefronts per head, each owning 32 of the 64 query rows; two wavefronts per
// SIMD (<= 256 registers), so the vector work of one overlaps the matrix
// instructions of the other.  Every product is a 32x32x16 MFMA:
//   S^T = K Q^T and dP^T = V dO^T, 32 keys at a time (lane: query l32 and 16
//   keys), so P and dS of a lane belong to one query row (its LSE and Delta
//   are per-lane scalars);
//   dQ^T += K^T dS^T, with dS^T packed to bf16 straight from the accumulator
//   layout as the B operand and K^T from transposed reads of the K tile (the
//   keys of both operands permuted the same way).
// K / V tiles are double-buffered in LDS: tile t + 1 is copied while tile t
// is processed, one barrier per tile.
// OUTER: the outer gate position (Sec. 4.1, Tab. 1 row 3): P carries no gate
// bias and the tile's gate g scales dP (dP = g dO V^T).
//
// KS (one head, four wavefronts): wavefront (kq, half) takes keys kq*32 ..
// +31 of every tile for its 32 query rows; the two key halves' dQ and
// P * dP sums are added in LDS at the end.  A one-head workgroup (per-head
// gates) then has four wavefronts on its 64 KB of K / V stages, so two such
// workgroups fill a CU's SIMDs twice.
template <int NH, bool PACKED, bool OUTER, bool KS = false>
__global__ void __launch_bounds__(NH * 128 * (KS ? 2 : 1), 2) bwd_dq_kernel(BwdArgs a) {
  static_assert(!KS || NH == 1, "the key split is for one-head workgroups");
  constexpr int NW = 2 * NH * (KS ? 2 : 1);
  __shared__ __attribute__((aligned(16))) bf16 s_k[2][TILE];
  __shared__ __attribute__((aligned(16))) bf16 s_v[2][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int half = w & 1;
  const int kq = KS ? (w >> 1) : 0;   // KS: this wave's key half of every tile

  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int chunk = unit % a.nchunk;
  const int rest = unit / a.nchunk;
  const int i = rest % a.C;
  const int bhk = rest / a.C;
  const int hk = bhk % a.Hkv;
  const int bb = bhk / a.Hkv;
  const int h = hk * a.G + a.head_base + chunk * NH + (KS ? 0 : (w >> 1));
  const long long row = ((long long)bb * a.Hs + h / a.Gs) * a.C + i;   // the head's gate row
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  const float* lgrow = a.lg + row * a.C;
  // workspace index of this lane's query row (padded order in every layout)
  const long long qr = ((long long)bb * a.Hq + h) * a.N + (long long)i * BLK + half * 32 + l32;

  // Variable-length batch: padding rows get Delta = 0 and -LSE = -inf in the
  // workspace, and dQ = 0 in the padded layout (a packed batch has no such
  // rows); a block without a valid row does nothing else (this return
  // precedes every copy and barrier and is uniform over the workgroup).
  constexpr bool packed = PACKED;   // packed variable-length batch (compile-time)
  const Span sp = seq_span(a, bb);
  const int nb = sp.n;
  if (i * BLK >= nb) {
    if (kq != 0) return;   // KS: the kq = 0 waves write the block
    if (g == 0) {
      a.delta[qr] = 0.0f;
      a.lsen[qr] = -INFINITY;
    }
    if (packed) return;
    bf16* dqp = a.dq + qr * HD + g * 4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(bf16x4*)(dqp + dt * 32 + q4 * 8) = bf16x4{(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
    return;
  }
  const bool row_valid = i * BLK + half * 32 + l32 < nb;
  // tensor rows of this lane's query (q, o, dO, dq) and its LSE entry; in a
  // packed batch the token is clamped to the sequence's last row
  const int tok = min(i * BLK + half * 32 + l32, nb - 1);
  const long long qt = packed ? (sp.start + tok) * a.Hq + h : qr;
  const long long ql = packed ? (long long)h * a.T + sp.start + tok : qr;
  const long long kv_stride = packed ? (long long)a.Hkv * HD : HD;

  auto load_tile = [&](int kb, int stg) {
    const long long t0 = packed ? ((sp.start + (long long)kb * BLK) * a.Hkv + hk) * HD
                                : ((long long)bhk * a.N + (long long)kb * BLK) * HD;
    const int rmax = packed ? min(BLK - 1, nb - 1 - kb * BLK) : BLK - 1;
    tile_to_lds<NW>(s_k[stg], a.k + t0, kv_stride, rmax, w, lane);
    tile_to_lds<NW>(s_v[stg], a.v + t0, kv_stride, rmax, w, lane);
  };
  const int ntiles = cnt + 1;
  load_tile(i, 0);
  // the row's selection (lane e: block of entry e), read up to the capacity
  // so that it goes out with the loads of Q, dO and O below instead of
  // waiting for the count (its gate gather follows the Delta computation)
  int selv = 0;
  float betav = 0.0f;
  {
    const int raw = lane < a.cap ? sel[lane] : 0;
    selv = lane < cnt ? raw : 0;
  }

  // Q^T and dO^T as B operands (lane: query row l32, dims ks*16 + g*8 .. +7);
  // dlt = rowsum(O * dO) over the row's two lanes (the Delta of dS in this
  // pass), dx = the row's sum of P * dP over every attended key (the same
  // quantity without the rounding of O; the key-major pass uses it)
  bf16x8 qf[8], dof[8];
  float part_d = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int d0 = ks * 16 + g * 8;
    qf[ks] = *(const bf16x8*)(a.q + qt * HD + d0);
    dof[ks] = *(const bf16x8*)(a.d_o + qt * HD + d0);
  }
  if (a.o_fp32) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float* op = (const float*)a.o + qt * HD + ks * 16 + g * 8;
      const f32x4 o0 = *(const f32x4*)op;
      const f32x4 o1 = *(const f32x4*)(op + 4);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        part_d += o0[x] * (float)dof[ks][x];
        part_d += o1[x] * (float)dof[ks][x + 4];
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 ob = *(const bf16x8*)((const bf16*)a.o + qt * HD + ks * 16 + g * 8);
#pragma unroll
      for (int x = 0; x < 8; ++x) part_d += (float)ob[x] * (float)dof[ks][x];
    }
  }
  const float dlt = sum2(part_d);
  const float lse2 = a.lse[ql] * kLog2e;
  float dx = 0.0f;

  f32x16 dqacc[4];   // dQ^T (lane: dims dt*32 + 8 (jj/4) + 4 g + jj%4, query l32)
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int x = 0; x < 16; ++x) dqacc[dt][x] = 0.0f;

  // transposed-read offsets of the K^T fragments (A operand of dQ^T, lane:
  // head dim dt*32 + l32, keys 16 sl + {4g .. 4g+3, 8+4g .. 8+4g+3})
  const int u = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  int tro[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      tro[dt][hh] = swz(g * 4 + (u >> 2) + 8 * hh, dt * 4 + dhalf * 2 + ((u >> 1) & 1)) + (u & 1) * 4;

  // One 64-key tile, as two halves of 32 keys: recompute S^T and dP^T, form
  // P and dS (packed to bf16 as the B operand of dQ^T: element jj -> k-slice
  // jj / 8, word (jj % 8) / 2), accumulate dQ^T and the row's P * dP.
  // The instruction order is pinned (sched_barrier): K / V fragments are read
  // two MFMAs ahead, and the first K^T fragments of the dQ^T product are read
  // before the vector work of P and dS, which hides their latency.  The
  // matrix sections run at raised wave priority: after each barrier the two
  // wavefronts of a SIMD fall into alternation, one issuing MFMAs while the
  // other does its vector work.
  auto ktr = [&](const bf16* Ks, int kh, int dt, int sl) {
    const bf16* kp = Ks + (kh * 32 + sl * 16) * HD;
    return join(ds_read_tr(kp + tro[dt][0]), ds_read_tr(kp + tro[dt][1]));
  };
  auto tile = [&](auto diag_tag, int stg, float beta) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    const bf16* Ks = s_k[stg];
    const bf16* Vs = s_v[stg];
    const float off = (OUTER ? 0.0f : beta) - lse2;
    const float gv = OUTER ? __builtin_amdgcn_exp2f(beta) : 1.0f;   // outer: the tile's gate
#pragma unroll
    for (int kk = 0; kk < (KS ? 1 : 2); ++kk) {
      const int kh = KS ? kq : kk;
      const int rr = kh * 32 + l32;
      f32x16 sc, dp;
#pragma unroll
      for (int x = 0; x < 16; ++x) { sc[x] = 0.0f; dp[x] = 0.0f; }
      bf16x8 ka[2], va[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        ka[ks] = *(const bf16x8*)(Ks + swz(rr, ks * 2 + g));
        va[ks] = *(const bf16x8*)(Vs + swz(rr, ks * 2 + g));
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sc = mfma32(ka[ks & 1], qf[ks], sc);
        dp = mfma32(va[ks & 1], dof[ks], dp);
        if (ks + 2 < 8) {
          ka[ks & 1] = *(const bf16x8*)(Ks + swz(rr, (ks + 2) * 2 + g));
          va[ks & 1] = *(const bf16x8*)(Vs + swz(rr, (ks + 2) * 2 + g));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 kt[2][2];   // K^T fragments of head-dim tiles dt, dt + 1
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) kt[d2][sl] = ktr(Ks, kh, d2, sl);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      uint32_t dsw[2][4];
#pragma unroll
      for (int jj = 0; jj < 16; jj += 2) {
        f32x2 pp;
        pp[0] = __builtin_amdgcn_exp2f(fmaf(sc[jj], a.c2, off));
        pp[1] = __builtin_amdgcn_exp2f(fmaf(sc[jj + 1], a.c2, off));
        if (DIAG) {   // causal mask: key > query -> P = 0
          const int key = kh * 32 + (jj >> 2) * 8 + g * 4 + (jj & 3);
          const int qrow = half * 32 + l32;
          if (key > qrow) pp[0] = 0.0f;
          if (key + 1 > qrow) pp[1] = 0.0f;
        }
        const float dp0 = OUTER ? dp[jj] * gv : dp[jj];
        const float dp1 = OUTER ? dp[jj + 1] * gv : dp[jj + 1];
        dx = fmaf(pp[0], dp0, dx);
        dx = fmaf(pp[1], dp1, dx);
        const f32x2 ds = {pp[0] * (dp0 - dlt), pp[1] * (dp1 - dlt)};
        dsw[jj >> 3][(jj & 7) >> 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(ds, bf16x2));
      }
      bf16x8 db[2];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
        db[sl] = __builtin_bit_cast(bf16x8, u32x4{dsw[sl][0], dsw[sl][1], dsw[sl][2], dsw[sl][3]});
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      // dQ^T: tiles dt = 0..3; the fragments of tile dt + 2 are read while
      // the MFMAs of tile dt run
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) dqacc[dt] = mfma32(kt[dt & 1][sl], db[sl], dqacc[dt]);
        if (dt + 2 < 4) {
#pragma unroll
          for (int sl = 0; sl < 2; ++sl) kt[dt & 1][sl] = ktr(Ks, kh, dt + 2, sl);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // the row's selection, 64 entries at a time, in registers (lane e: block
  // sel[e0 + e] and its log gate in log2 units), read with readlane; both
  // loads complete inside the (rarely taken) reload branch, so that no load
  // is in flight where the branch joins the tile loop
  auto load_sel = [&](int e0) {
    const int e = e0 + lane;
    selv = e < cnt ? sel[e] : 0;
    betav = (e < cnt && !a.hard) ? lgrow[selv] * kLog2e : 0.0f;   // hard gates: unit
    settle(selv);
    settle(betav);
  };
  betav = (lane < cnt && !a.hard) ? lgrow[selv] * kLog2e : 0.0f;   // hard gates: unit
  settle(selv);
  settle(betav);

  wait_vm();
  __syncthreads();
  float nbeta = 0.0f;   // log gate of the tile in the other stage
  if (ntiles > 1) {
    load_tile(lane_value(selv, 0), 1);
    nbeta = lane_value(betav, 0);
  }
  tile(std::true_type{}, 0, 0.0f);   // diagonal block (causal, gate 0)
  wait_vm();
  __syncthreads();
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
  if (KS) {
    // add the kq = 1 waves' dQ^T and P * dP sums into the kq = 0 waves'
    // (K stages: dQ^T, lane-major 16-byte vectors; V stage 0: the sums); the
    // loop's last barrier has retired every read of the stages
    f32x4* xo = (f32x4*)&s_k[0][0] + half * 16 * 64 + lane;
    float* xd = (float*)&s_v[0][0] + half * 64 + lane;
    if (kq == 1) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xo[(dt * 4 + q4) * 64] = f32x4{dqacc[dt][q4 * 4], dqacc[dt][q4 * 4 + 1], dqacc[dt][q4 * 4 + 2],
                                         dqacc[dt][q4 * 4 + 3]};
      *xd = dx;
    }
    __syncthreads();
    if (kq == 1) return;
    dx += *xd;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 ob = xo[(dt * 4 + q4) * 64];
#pragma unroll
        for (int y = 0; y < 4; ++y) dqacc[dt][q4 * 4 + y] += ob[y];
      }
  }
  const float dsum = sum2(dx);
  if (g == 0) {
    a.delta[qr] = row_valid ? dsum : 0.0f;
    a.lsen[qr] = row_valid ? -lse2 : -INFINITY;
  }
  // the row's selection into the key-major column bit masks (zeroed before
  // this kernel): bit i*nsh + sl of column (batch, kv head, block m) for each
  // selected m, set by one wavefront per gate row (the first row half of the
  // score head's first query head), after its last tile so that these
  // atomics hold up no wait of the tile loop
  if (half == 0 && h % a.Gs == 0) {
    const int code = i * a.nsh + (h / a.Gs - hk * a.nsh);
    const uint32_t bit = 1u << (code & 31);
    uint32_t* cm = a.colmask + (long long)bhk * a.C * a.W + (code >> 5);
    for (int e = lane; e < cnt; e += 64) atomicOr(cm + (long long)sel[e] * a.W, bit);
  }

  // dQ = scale * dQacc (lane: query l32, dims dt*32 + q4*8 + 4 g .. +3)
  if (packed && !row_valid) return;   // the row belongs to no sequence of this batch
  bf16* dqp = a.dq + qt * HD + g * 4;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 r;
#pragma unroll
      for (int y = 0; y < 4; ++y) r[y] = (bf16)(row_valid ? dqacc[dt][q4 * 4 + y] * a.scale : 0.0f);
      *(bf16x4*)(dqp + dt * 32 + q4 * 8) = r;
    }
}

// ---------------------------------------------------------------------------
// hard Top-K gates: gate gradients of the dropped blocks
// ---------------------------------------------------------------------------
// Straight-through estimator (Sec. 4.1 "Ranking preservation", Eq. 7): the
// gate gradient of a dropped historical block m of query block i is the
// attention mass its keys would get under the selected set's normaliser,
// exp(z - lse), times (dP - Delta), summed over the block's keys, the query
// block's rows and the score head's query heads.  One workgroup per gate row
// (batch, score head s, query block i): four wavefronts = two heads x two
// 32-row halves per round, rounds over the row's Gs heads; the dropped
// blocks (m < i, not selected) stream through a double-buffered LDS tile;
// per tile a wavefront sums P (dP - Delta) over its rows and the tile's keys
// (S^T = K Q^T and dP^T = V dO^T on 32x32x16 MFMAs, one query row per lane),
// with P = exp2(S c2 - LSE log2 e) from the query-major pass's -LSE copy
// (-inf on padding rows, so they add nothing) and Delta from the same pass.
// The four partial sums meet in LDS and are added into the row's per-block
// accumulator in a fixed order (deterministic).
constexpr size_t kSteStaticLds = 2 * 2 * TILE * sizeof(bf16) + 2 * 4 * sizeof(float);
__host__ __device__ constexpr size_t ste_dynamic_lds(int C) {
  return sizeof(uint32_t) * (size_t)((C + 31) / 32) + sizeof(float) * (size_t)C;
}
static_assert(kSteStaticLds + ste_dynamic_lds(8192) <= 160 * 1024,
              "the dropped-block pass fits the largest supported block count");

__global__ void __launch_bounds__(256) ste_mfma_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 s_k[2][TILE];
  __shared__ __attribute__((aligned(16))) bf16 s_v[2][TILE];
  __shared__ float part[2][4];
  extern __shared__ float s_dyn[];   // selection bitmask (C / 32 words), then C accumulators
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int half = w & 1;

  const long long row = blockIdx.x;   // (batch * Hs + s) * C + i
  const int i = (int)(row % a.C);
  const long long bs = row / a.C;
  const int sh = (int)(bs % a.Hs);
  const int bb = (int)(bs / a.Hs);
  const int hk = sh * a.Gs / a.G;
  const long long bhk = (long long)bb * a.Hkv + hk;
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  const Span sp = seq_span(a, bb);
  const bool packed = a.cu != nullptr;
  // no dropped block (every historical block selected) or no valid query:
  // nothing to write (uniform; before any copy or barrier)
  if (i - cnt <= 0 || i * BLK >= sp.n) return;

  const int words = (a.C + 31) >> 5;
  uint32_t* selmask = (uint32_t*)s_dyn;
  float* accm = s_dyn + words;
  for (int x = tid; x < words; x += blockDim.x) selmask[x] = 0u;
  for (int x = tid; x < i; x += blockDim.x) accm[x] = 0.0f;
  __syncthreads();
  for (int e = tid; e < cnt; e += blockDim.x) {
    const int m = min(max(sel[e], 0), a.C - 1);
    atomicOr(&selmask[m >> 5], 1u << (m & 31));
  }
  __syncthreads();
  // the first dropped block after m (i when there is none); uniform
  auto next_dropped = [&](int m) {
    for (++m; m < i; ++m)
      if (((selmask[m >> 5] >> (m & 31)) & 1u) == 0u) return m;
    return i;
  };
  const long long kv_stride = packed ? (long long)a.Hkv * HD : HD;
  auto load_tile = [&](int kb, int stg) {   // dropped blocks lie before i: full tiles
    const long long t0 = packed ? ((sp.start + (long long)kb * BLK) * a.Hkv + hk) * HD
                                : (bhk * a.N + (long long)kb * BLK) * HD;
    tile_to_lds<4>(s_k[stg], a.k + t0, kv_stride, BLK - 1, w, lane);
    tile_to_lds<4>(s_v[stg], a.v + t0, kv_stride, BLK - 1, w, lane);
  };

  const int m0 = next_dropped(-1);
  const int rounds = (a.Gs + 1) / 2;
  for (int r = 0; r < rounds; ++r) {
    const int hl = 2 * r + (w >> 1);          // head of this wavefront within the score head
    const bool on = hl < a.Gs;                 // uniform per wavefront
    const int h = sh * a.Gs + (on ? hl : 0);
    const int tok = min(i * BLK + half * 32 + l32, sp.n - 1);
    const long long wsr = ((long long)bb * a.Hq + h) * a.N + (long long)i * BLK + half * 32 + l32;
    const long long qt = packed ? (sp.start + tok) * a.Hq + h : wsr;
    bf16x8 qf[8], dof[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *(const bf16x8*)(a.q + qt * HD + ks * 16 + g * 8);
      dof[ks] = *(const bf16x8*)(a.d_o + qt * HD + ks * 16 + g * 8);
    }
    const float nl = a.lsen[wsr];      // -LSE log2(e), -inf on padding rows
    const float dlt = a.delta[wsr];    // sum of P dP over the row's attended keys
    load_tile(m0, 0);
    wait_vm();
    __syncthreads();
    int m = m0, stg = 0, par = 0;
    while (m < i) {
      const int mn = next_dropped(m);
      if (mn < i) load_tile(mn, stg ^ 1);   // prefetch the next dropped block
      float acc = 0.0f;
      if (on) {
        const bf16* Ks = s_k[stg];
        const bf16* Vs = s_v[stg];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int rr = kh * 32 + l32;
          f32x16 sc, dp;
#pragma unroll
          for (int x = 0; x < 16; ++x) { sc[x] = 0.0f; dp[x] = 0.0f; }
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            sc = mfma32(*(const bf16x8*)(Ks + swz(rr, ks * 2 + g)), qf[ks], sc);
            dp = mfma32(*(const bf16x8*)(Vs + swz(rr, ks * 2 + g)), dof[ks], dp);
          }
#pragma unroll
          for (int jj = 0; jj < 16; ++jj)
            acc = fmaf(__builtin_amdgcn_exp2f(fmaf(sc[jj], a.c2, nl)), dp[jj] - dlt, acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) part[par][w] = acc;
      wait_vm();
      __syncthreads();   // partials of block m; block mn staged
      if (tid == 0) accm[m] += ((part[par][0] + part[par][1]) + part[par][2]) + part[par][3];
      m = mn;
      stg ^= 1;
      par ^= 1;
    }
    __syncthreads();   // the next round reuses the tile buffers
  }
  float* drow = a.dlg + row * a.C;
  for (int x = tid; x < i; x += blockDim.x)
    if (((selmask[x >> 5] >> (x & 31)) & 1u) == 0u) drow[x] = accm[x];
}

// ---------------------------------------------------------------------------
// selection transpose: column lists
// ---------------------------------------------------------------------------
__global__ void fill_zero_kernel(uint32_t* p, long long n) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    p[e] = 0u;
}

__global__ void count_kernel(BwdArgs a) {
  const long long col = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= a.ncol) return;
  int L = a.nsh;  // the diagonal block, once per score head
  for (int w = 0; w < a.W; ++w) L += __popc(a.colmask[col * a.W + w]);
  a.collen[col] = L;
  a.chunk_hist[col] = 0;   // the order buckets' counters (chunk_count_kernel)
}

// exclusive prefix sums of the column lengths and chunk counts (one workgroup)
__global__ void __launch_bounds__(1024) scan_kernel(BwdArgs a) {
  __shared__ int s_len[1024], s_chk[1024];
  const int t = threadIdx.x;
  const long long per = (a.ncol + 1023) / 1024;
  const long long beg = min((long long)t * per, a.ncol);
  const long long end = min(beg + per, a.ncol);
  int sl = 0, sc = 0;
  for (long long c = beg; c < end; ++c) {
    const int L = a.collen[c];
    sl += L;
    sc += (L + a.cc - 1) / a.cc;
  }
  s_len[t] = sl;
  s_chk[t] = sc;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {   // Hillis-Steele inclusive scan
    const int xl = t >= off ? s_len[t - off] : 0;
    const int xc = t >= off ? s_chk[t - off] : 0;
    __syncthreads();
    s_len[t] += xl;
    s_chk[t] += xc;
    __syncthreads();
  }
  int ol = s_len[t] - sl, oc = s_chk[t] - sc;
  for (long long c = beg; c < end; ++c) {
    const int L = a.collen[c];
    a.coloff[c] = ol;
    a.chunkoff[c] = oc;
    ol += L;
    oc += (L + a.cc - 1) / a.cc;
  }
  if (t == 1023) {
    a.coloff[a.ncol] = s_len[1023];
    a.chunkoff[a.ncol] = s_chk[1023];
  }
}

__global__ void __launch_bounds__(256) fill_lists_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const long long col = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= a.ncol) return;
  const int j = (int)(col % a.C);
  int32_t* out = a.collist + a.coloff[col];
  for (int x = lane; x < a.nsh; x += 64) out[x] = j * a.nsh + x;   // the diagonal entries
  int run = a.nsh;
  for (int w0 = 0; w0 < a.W; w0 += 64) {
    const int wi = w0 + lane;
    uint32_t bits = wi < a.W ? a.colmask[col * a.W + wi] : 0u;
    const int c = __popc(bits);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    int pos = run + incl - c;
    while (bits) {
      const int b = __builtin_ctz(bits);
      out[pos++] = wi * 32 + b;
      bits &= bits - 1u;
    }
    run += __shfl(incl, 63, 64);
  }
}

// Column chunk g -> (column, chunk index within the column).
__device__ __forceinline__ long long chunk_column(const BwdArgs& a, int g) {
  long long lo = 0, hi = a.ncol;   // chunkoff[lo] <= g < chunkoff[hi]
  while (hi - lo > 1) {
    const long long mid = (lo + hi) >> 1;
    if (a.chunkoff[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

// Order of the key-major work: chunks sorted by (batch, kv head, order
// bucket).  The bucket of a chunk is the first query block it reads, so that
// workgroups that run at the same time stream nearby query blocks and share
// their Q / dO rows through the L2 / MALL.  Chunks that start in the last
// third of the sequence are bucketed by length instead (longest first; within
// one length, by first query block in R / cc coarse steps): there the lists
// run out, and a long chunk that starts late would run on alone after the
// others have finished.  (Same-box A/B at 32k: key-major kernel 2-3 % faster
// than with first-block buckets throughout.)  The order only schedules work;
// every result is reduced in a fixed order.
__device__ __forceinline__ long long chunk_key(const BwdArgs& a, long long col, int first, int ne) {
  const int T = a.C - a.C / 3;
  const int R = a.C - T;
  int k = first;
  if (first >= T && R > 1) {
    const int sb = max(1, R / a.cc);
    const int cls = a.cc - min(ne, a.cc);   // 0: the longest chunks
    k = T + min(R - 1, cls * sb + (int)((long long)(first - T) * sb / R));
  }
  return col - col % a.C + k;   // (batch, kv head) row base + bucket
}

// rank of each chunk inside its order bucket
__global__ void chunk_count_kernel(BwdArgs a) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= a.chunkoff[a.ncol]) return;
  const long long col = chunk_column(a, g);
  const int c = g - a.chunkoff[col];
  const int first = a.collist[a.coloff[col] + c * a.cc] / a.nsh;   // its first query block
  const int ne = min(a.collen[col], c * a.cc + a.cc) - c * a.cc;
  const long long key = chunk_key(a, col, first, ne);
  a.chunk_rank[g] = atomicAdd(&a.chunk_hist[key], 1);
}

// exclusive prefix sum of n ints in place (one workgroup); x[n] = total
__global__ void __launch_bounds__(1024) scan_ints_kernel(int32_t* x, long long n) {
  __shared__ int s[1024];
  const int t = threadIdx.x;
  const long long per = (n + 1023) / 1024;
  const long long beg = min((long long)t * per, n);
  const long long end = min(beg + per, n);
  int sum = 0;
  for (long long e = beg; e < end; ++e) sum += x[e];
  s[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int y = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += y;
    __syncthreads();
  }
  int run = s[t] - sum;
  for (long long e = beg; e < end; ++e) {
    const int v = x[e];
    x[e] = run;
    run += v;
  }
  if (t == 1023) x[n] = s[1023];
}

// Writes the descriptor of chunk g at its place in the order, indexed by the
// hardware workgroup id that runs it (the inverse of the key-major kernel's
// XCD remap): the key-major workgroup then finds its work with one load
// instead of a binary search over the chunk offsets.
__global__ void chunk_scatter_kernel(BwdArgs a) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  const int total = a.chunkoff[a.ncol];
  if (g >= total) return;
  const long long col = chunk_column(a, g);
  const int c = g - a.chunkoff[col];
  const int nch = a.chunkoff[col + 1] - a.chunkoff[col];
  const int e0 = c * a.cc;
  const int first = a.collist[a.coloff[col] + e0] / a.nsh;
  const int ne = min(a.collen[col], e0 + a.cc) - e0;
  const long long key = chunk_key(a, col, first, ne);
  const int pos = a.chunk_hist[key] + a.chunk_rank[g];
  int32_t* d = a.chunk_desc + 4 * (long long)xcd_unmap(pos, total);
  d[0] = g;
  d[1] = (int)col;
  d[2] = a.coloff[col] + e0;
  d[3] = ne | (nch == 1 ? (1 << 30) : 0);
}

// ---------------------------------------------------------------------------
// key-major pass: dK, dV and the block log-gate gradient
// ---------------------------------------------------------------------------
// 32x32x16 operand layouts (lane l, g = l / 32):
//   A: row l % 32, k = 8 g .. 8 g + 7;   B: column l % 32, same k;
//   C: column l % 32, rows 8 (jj / 4) + 4 g + jj % 4 for jj = 0..15.
// The C fragment of S (rows x keys) feeds the B operand of the row
// contraction directly: its elements 8 sl .. 8 sl + 7 are rows
// 16 sl + {4 g .. 4 g + 3, 8 + 4 g .. 8 + 4 g + 3}, and the transposed reads of
// the staged rows use the same row order.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int XS_BYTES = 32 * HD * 2;               // 32 staged rows
constexpr int SLOT_BYTES = 256 + XS_BYTES;           // one statistic (64 floats), then the rows
constexpr int Q_SLOTS = 5, O_SLOTS = 3;
constexpr int QRING = 0;
constexpr int ORING = QRING + Q_SLOTS * SLOT_BYTES;

// Keeps the computation of x at this point of the instruction stream: the
// vector-ALU work that is meant to overlap a matrix instruction would
// otherwise be sunk to its first use.
template <typename T>
__device__ __forceinline__ void pin(T& x) { __asm__ volatile("" : "+v"(x)); }

// Element offset of 16-byte chunk c of row r in a staged 32 x 128 tile
// (slot16 swizzle).
__device__ __forceinline__ int xsw(int r, int c) { return r * HD + ((c ^ slot16(r)) << 3); }


// One workgroup = four wavefronts = one column chunk (key block j, up to
// a.cc query blocks), streamed in steps of 32 query rows of one head
// (n steps: entry e, head h, half x -> step 2 (e G + h) + x).  Pair kh (waves
// 2 kh, 2 kh + 1) owns keys kh*32 .. kh*32 + 31 of the block and splits the
// work by tensor:
//   wave A (role 0): S = Q K^T -> P, and dV^T += dO^T P   (its K rows resident)
//   wave B (role 1): dP = dO V^T -> dS = P (dP - Delta), dK^T += Q^T dS
//                    (its V rows resident)
// Each wavefront holds 32 keys (about 225 registers), so two run per SIMD and
// one's vector work overlaps the other's matrix instructions; every product
// is a 32x32x16 MFMA.
//
// Software pipeline (window s lies between barriers s - 1 and s):
//   A: S_{s+1} (matrix core) overlapped with P_s = exp(S_s ...) (vector ALU),
//      then dV_s += dO_s^T P_s;  P_s is published (fp16) at barrier s.
//   B: dP_s (matrix core) overlapped with dS_{s-1} (vector ALU), then
//      dK_{s-1} += Q_{s-1}^T dS_{s-1}.
// A step's rows reach LDS by asynchronous global -> LDS copies into two rings
// shared by the pairs: the A waves copy the Q rows (half each; key half 0
// also Delta) into a 5-slot ring (step t is read in windows t - 1 .. t + 1),
// the B waves the dO rows (and LSE) into a 3-slot ring (read in window t),
// two windows before first use, spread between the contraction's MFMAs, with
// one LDS base (M0) per step; every wavefront waits for its own copies before
// the barrier that publishes them.  The Q / dO operand
// fragments are read two MFMAs ahead.  B's per-entry dS sums of the two key
// halves meet in LDS and are added in a fixed order after the loops
// (deterministic).
constexpr int PX4_BYTES = 32 * 32 * 2;                       // P of one step, one key half (fp16)
constexpr int PBUF4 = ORING + O_SLOTS * SLOT_BYTES;
constexpr int ITAB4 = PBUF4 + 2 * 2 * PX4_BYTES;             // [key half][step parity]
constexpr int GTAB4 = ITAB4 + 2 * kColChunkMax * 4;          // itab + btab
constexpr int KV4_LDS = GTAB4 + 2 * kColChunkMax * 4;        // dLogG partials [key half][entry]
static_assert(2 * KV4_LDS <= 160 * 1024, "two workgroups per CU");

// Ring barrier: this wavefront's LDS accesses and all but its newest copies
// (one step's: five for key half 0, four for key half 1) are complete, then
// s_barrier.  (__syncthreads would also wait for the newest copies, which
// are meant to stay in flight.)
__device__ __forceinline__ void ring_barrier(int kh) {
  if (kh == 0) __asm__ volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else __asm__ volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS address of the next global -> LDS copies (M0); the 1-wait-state
// hazard before a copy is covered here.
__device__ __forceinline__ void set_lds_m0(unsigned lds) {
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0" :: "s"(__builtin_amdgcn_readfirstlane(lds))
                   : "memory", "m0");
}
// 16 bytes per lane from base + voff + OFF to LDS M0 + OFF + 16 lane (the
// instruction offset moves both addresses).
template <int OFF>
__device__ __forceinline__ void dma16_at(const void* base, unsigned voff) {
  __asm__ volatile("global_load_lds_dwordx4 %0, %1 offset:%2" :: "v"(voff), "s"(uniform_ptr(base)),
                   "i"(OFF) : "memory");
}

// PACKED: packed variable-length batch (a compile-time switch, so the copies
// of the fixed-length and padded layouts keep their one-base form).
// OUTER: the outer gate position (Sec. 4.1, Tab. 1 row 3): P carries no gate
// bias, dV takes g P, dS = P (g dP - Delta) and dLogG sums P g dP.
template <bool PACKED, bool OUTER>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[KV4_LDS];
  int32_t* itab = (int32_t*)(smem + ITAB4);   // query block of each chunk entry
  float* btab = (float*)(itab + kColChunkMax);   // its log gate (log2 units; 0 on the diagonal)
  float* gtab = (float*)(smem + GTAB4);       // [key half][entry] dS sums

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wv & 1;   // 0: S / P / dV, 1: dP / dS / dK (wave-uniform)
  const int kh = wv >> 1;    // key half
  const int g = lane >> 5;
  const int l32 = lane & 31;

  // this workgroup's chunk (descriptor written by chunk_scatter_kernel at
  // this hardware id; scalar loads, both in flight together)
  typedef __attribute__((address_space(4))) const int32_t cint;
  const int total = *(cint*)(a.chunkoff + a.ncol);
  const cint* dsc = (cint*)(a.chunk_desc + 4 * (long long)blockIdx.x);
  const int gch = dsc[0], dcol = dsc[1], loff = dsc[2], dne = dsc[3];
  if ((int)blockIdx.x >= total) return;
  const long long col = dcol;
  const int ne = dne & ((1 << 30) - 1);
  const bool only_chunk = (dne >> 30) & 1;
  // column col = (batch, kv head, key block j); an entry is (query block i,
  // score head sl of the kv head) with its own gate row, covering the score
  // head's G = Gs query heads (the kv group with group gates, one head with
  // per-head gates)
  const int j = (int)(col % a.C);
  const long long bhk = col / a.C;
  const int hk = (int)(bhk % a.Hkv);
  const int bb = (int)(bhk / a.Hkv);
  const int G = a.Gs;   // query heads per entry
  constexpr bool packed = PACKED;
  const Span sp = seq_span(a, bb);
  // A packed batch has no rows for a key block past its sequence's end (no
  // selecting row, only the diagonal entry with no valid query): nothing to
  // do.  Uniform over the workgroup, before any copy or barrier.
  if (packed && j * BLK >= sp.n) return;

  // resident B operand of S (A: K_j) or dP (B: V_j): key kh*32 + l32,
  // dims ds*16 + g*8 .. +7 (in flight with the column list below; the first
  // products wait for them)
  bf16x8 kf[8];
  {
    const int key = j * BLK + kh * 32 + l32;
    const long long kr = packed ? (sp.start + min(key, sp.n - 1)) * a.Hkv + hk
                                : bhk * a.N + key;
    const bf16* t = (role == 0 ? a.k : a.v) + kr * HD;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) kf[ds] = *(const bf16x8*)(t + ds * 16 + g * 8);
  }

  // The entry table (itab, btab) written here by wavefront 0 is read by the
  // other wavefronts only after their first ring barrier (an s_barrier after
  // lgkmcnt(0)), so the first row copies go out without a barrier of their
  // own, as soon as the column list has arrived.
  long long rowbase = 0;   // per entry: workspace row of (query block, head 0) (padded order)
  long long prow = 0;      // packed batch: tensor row of (query block, head 0)
  int vrem = 0;            // packed batch: valid rows of the entry's query block
  int diag_e = 0;   // this lane's entry is a diagonal one (query block j)
  if (lane < ne) {
    const int code = a.collist[loff + lane];
    const int i = code / a.nsh;
    const long long bs = bhk * a.nsh + code % a.nsh;   // gate-table row base: batch * Hs + s
    const int sh = (int)(bs % a.Hs);
    if (wv == 0) {
      itab[lane] = code;
      btab[lane] = (i == j || a.hard) ? 0.0f : a.lg[(bs * a.C + i) * a.C + j] * kLog2e;
    }
    rowbase = ((long long)bb * a.Hq + sh * G) * a.N + (long long)i * BLK;
    prow = (sp.start + (long long)i * BLK) * a.Hq + sh * G;
    vrem = sp.n - i * BLK;
    diag_e = i == j;
  }
  // the diagonal entries (one per score head) lead the column's list
  const int ndiag = __builtin_popcountll(__builtin_amdgcn_ballot_w64(diag_e != 0));


  const int n = 2 * ne * G;   // steps: entry e, head h, half x -> step 2 (e G + h) + x
  const int nslots = role == 0 ? Q_SLOTS : O_SLOTS;
  char* const ring = smem + (role == 0 ? QRING : ORING);
  const bf16* src = role == 0 ? a.q : a.d_o;
  const float* stat = role == 0 ? a.delta : a.lsen;
  // this lane's 16 bytes of copy q: rows (kh*4 + q)*4 .. +3, less the
  // q * 1024 that the instruction offset adds (rows >= 4 q, so >= 0)
  unsigned voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (kh * 4 + q) * 4 + (lane >> 4);
    voff[q] = (unsigned)(row * HD + (((lane & 15) ^ slot16(row)) << 3)) * 2 - q * 1024;
  }
  const unsigned soff = (unsigned)l32 * 4;
  int ct = 0, ce = 0, chh = 0, cx = 0, cslot = 0;
  const unsigned ring_lds = lds_addr(ring);
  // packed batch: rows of the entry's block are Hq * HD apart; copy q of a
  // step takes block rows cx*32 + (kh*4 + q)*4 + lane/16, clamped to the
  // block's last valid row (vr = its valid rows)
  struct Copy { const bf16* rows; const float* st; unsigned lds; int cx, vr; };
  auto prepare = [&]() -> Copy {
    const long long rbase = (long long)(unsigned)__builtin_amdgcn_readlane((int)rowbase, ce) |
                            ((long long)__builtin_amdgcn_readlane((int)(rowbase >> 32), ce) << 32);
    const long long r0 = rbase + (long long)(unsigned)(chh * a.N + cx * 32);
    Copy cp{src + r0 * HD, stat + r0, ring_lds + (unsigned)(cslot * SLOT_BYTES), cx, 0};
    if (packed) {
      const long long pb = (long long)(unsigned)__builtin_amdgcn_readlane((int)prow, ce) |
                           ((long long)__builtin_amdgcn_readlane((int)(prow >> 32), ce) << 32);
      cp.rows = src + (pb + chh) * HD;   // row 0 of the entry's block, head chh
      cp.vr = __builtin_amdgcn_readlane(vrem, ce);
    }
    cslot = cslot + 1 == nslots ? 0 : cslot + 1;
    if (++ct < n) {
      cx ^= 1;
      if (cx == 0 && ++chh == G) { chh = 0; ++ce; }
    }
    return cp;
  };
  // copies per step: four 1 KB row groups per wavefront (one M0 for the
  // four, placed by the instruction offsets), and the statistic (key half 0)
  auto issue = [&](const Copy& cp, int q) {
    if (packed) {   // one LDS base per copy; per-lane clamped rows
      if (q < 4) {
        const int row = (kh * 4 + q) * 4 + (lane >> 4);
        const int br = min(cp.cx * 32 + row, cp.vr - 1);
        const unsigned vo = (unsigned)((long long)br * a.Hq * HD + (((lane & 15) ^ slot16(row)) << 3)) * 2;
        dma16s(cp.rows, vo, cp.lds + 256 + (kh * 4 + q) * 1024);
      } else if (kh == 0) {
        dma4s(cp.st, soff, cp.lds);
      }
      return;
    }
    switch (q) {
      case 0:
        set_lds_m0(cp.lds + 256 + kh * 4096);
        dma16_at<0>(cp.rows, voff[0]);
        break;
      case 1: dma16_at<1024>(cp.rows, voff[1]); break;
      case 2: dma16_at<2048>(cp.rows, voff[2]); break;
      case 3: dma16_at<3072>(cp.rows, voff[3]); break;
      default:
        if (kh == 0) dma4s(cp.st, soff, cp.lds);
        break;
    }
  };
  auto copy_next = [&]() {
    const Copy cp = prepare();
#pragma unroll
    for (int q = 0; q < 5; ++q) issue(cp, q);
  };
  // rows of ring slot k (its statistic sits in the 256 bytes before them)
  auto qring = [&](int k) -> char* { return smem + QRING + k * SLOT_BYTES + 256; };
  auto oring = [&](int k) -> char* { return smem + ORING + k * SLOT_BYTES + 256; };
  auto inc = [](int k, int m) { return k + 1 == m ? 0 : k + 1; };

  f32x16 acc[4];   // A: dV^T, B: dK^T; lane: key kh*32 + l32, dims dt*32 + 8 (jj/4) + 4 g + jj%4
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int x = 0; x < 16; ++x) acc[dt][x] = 0.0f;

  const int u = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  const int tr_r = g * 4 + (u >> 2);
  int tro[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int h = 0; h < 2; ++h) tro[dt][h] = xsw(tr_r + 8 * h, dt * 4 + dhalf * 2 + ((u >> 1) & 1)) + (u & 1) * 4;
  auto tr_frag = [&](const char* rows, int dt, int sl) -> bf16x8 {
    const bf16* xs = (const bf16*)rows;
    return join(ds_read_tr(xs + tro[dt][0] + sl * 16 * HD), ds_read_tr(xs + tro[dt][1] + sl * 16 * HD));
  };
  // row contraction into the accumulators (8 MFMAs); the transposed
  // fragments are read two MFMAs ahead; after MFMA m the work per_mfma(m)
  // (raised wave priority: the other wavefront of the SIMD, in its vector
  // section, then fills the gaps between these MFMAs)
  auto contract = [&](const char* rows, const bf16x8 (&bop)[2], auto&& per_mfma) {
    bf16x8 ta[2];
    ta[0] = tr_frag(rows, 0, 0);
    ta[1] = tr_frag(rows, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int dt = m >> 1, sl = m & 1;
      acc[dt] = mfma32(ta[m & 1], bop[sl], acc[dt]);
      if (m + 2 < 8) ta[m & 1] = tr_frag(rows, (m + 2) >> 1, (m + 2) & 1);
      per_mfma(m);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto read_stat = [&](const char* sl, float (&st)[16]) {
    const float* sp = (const float*)(sl - 256);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x4 v = *(const f32x4*)(sp + t * 8 + g * 4);
#pragma unroll
      for (int y = 0; y < 4; ++y) st[t * 4 + y] = v[y];
    }
  };
  auto pbuf = [&](int t) -> _Float16* { return (_Float16*)(smem + PBUF4 + (kh * 2 + (t & 1)) * PX4_BYTES); };
  // S (A) or dP (B) of the rows in slot sl: 8 MFMAs, row fragments read two
  // ahead; after MFMA m the vector work per_mfma(m) of the previous step
  auto rows_product_with = [&](const char* sl, f32x16& out, auto&& per_mfma) {
    const bf16* xs = (const bf16*)sl;
    bf16x8 qa[2];
    qa[0] = *(const bf16x8*)(xs + xsw(l32, 0 * 2 + g));
    qa[1] = *(const bf16x8*)(xs + xsw(l32, 1 * 2 + g));
#pragma unroll
    for (int x = 0; x < 16; ++x) out[x] = 0.0f;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      out = mfma32(qa[ds & 1], kf[ds], out);
      if (ds + 2 < 8) qa[ds & 1] = *(const bf16x8*)(xs + xsw(l32, (ds + 2) * 2 + g));
      per_mfma(ds);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // A, window s: S_{s+1} (rows in qn) interleaved with P_s = exp2(c2 S_s +
  // beta - lse) (LSE in os), then dV_s += dO_s^T P_s; P_s also goes to LDS
  // (fp16) for B.  HALF: the step's half of its query block.
  const int key = kh * 32 + l32;
  // The statistic of the O ring is -LSE log2(e) per query row, written by
  // the query-major pass (-inf on padding rows of a variable-length batch, so
  // they get P = 0 and add nothing to dV, dK and dLogG).
  auto window_a = [&](auto diag_tag, auto half_tag, const char* qn, const char* os, _Float16* px,
                      float beta, const f32x16& sprev, f32x16& snext) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    constexpr int hrow = decltype(half_tag)::value * 32;
    float nl[16];
    read_stat(os, nl);
    if (!OUTER) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) nl[jj] += beta;
    }
    const float gv = OUTER ? __builtin_amdgcn_exp2f(beta) : 1.0f;   // outer: the entry's gate
    bf16x8 bop[2];
    f16x8 ph[2];
    rows_product_with(qn, snext, [&](int m) {
      float e2[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int jj = m * 2 + x;
        float e = __builtin_amdgcn_exp2f(fmaf(sprev[jj], a.c2, nl[jj]));
        if (DIAG && key > hrow + (jj >> 2) * 8 + g * 4 + (jj & 3)) e = 0.0f;
        e2[x] = e;
      }
      const int h2 = m >> 2, x0 = (m & 3) * 2;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        bop[h2][x0 + x] = (bf16)(OUTER ? e2[x] * gv : e2[x]);   // outer: dV takes g P
        ph[h2][x0 + x] = (_Float16)e2[x];
      }
      pin(bop[h2]);
      pin(ph[h2]);
    });
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) *(f16x8*)(px + (h2 * 64 + lane) * 8) = ph[h2];
    const Copy cp = prepare();
    contract(os, bop, [&](int m) { if (m < 5) issue(cp, m); });   // dV_s, this window's copies
  };
  // B: dS = P (dP - Delta) of the previous step (Delta and Q rows in qs, P
  // in px) as the bf16 B operand, element pair m after MFMA m of the next
  // dP, then dK += Q^T dS.  gsum collects the step's dS (fma with a zero
  // addend and the fp16 operand: one mixed-precision fma).
  auto window_b = [&](const char* on, const char* qs, const _Float16* px, const f32x16& dprev,
                      f32x16& dcur, float& gsum, float gv) {
    float dl[16];
    read_stat(qs, dl);
    f16x8 ph[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) ph[h2] = *(const f16x8*)(px + (h2 * 64 + lane) * 8);
    bf16x8 bop[2];
    rows_product_with(on, dcur, [&](int m) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int jj = m * 2 + x;
        const float pj = (float)ph[jj >> 3][jj & 7];
        const float dpj = OUTER ? dprev[jj] * gv : dprev[jj];
        const float ds = fmaf(pj, dpj - dl[jj], 0.0f);
        gsum = OUTER ? fmaf(pj, dpj, gsum) : gsum + ds;   // outer: dLogG sums P g dP
        bop[jj >> 3][jj & 7] = (bf16)ds;
      }
      pin(bop[m >> 2]);
    });
    const Copy cp = prepare();
    contract(qs, bop, [&](int m) { if (m < 5) issue(cp, m); });   // dK, this window's copies
  };

  f32x16 r0, r1;
  if (role == 0) {
    copy_next();
    copy_next();
    copy_next();
    ring_barrier(kh);   // Q of steps 0, 1 landed
    rows_product_with(qring(0), r0, [](int) {});   // S_0
    int qk = 1, ok = 0;
    const int nd = 2 * G * ndiag;
#pragma unroll 1
    for (int s = 0; s < nd; s += 2) {
      window_a(std::true_type{}, std::integral_constant<int, 0>{}, qring(qk), oring(ok), pbuf(0), 0.0f, r0, r1);
      ring_barrier(kh);
      qk = inc(qk, Q_SLOTS); ok = inc(ok, O_SLOTS);
      window_a(std::true_type{}, std::integral_constant<int, 1>{}, qring(qk), oring(ok), pbuf(1), 0.0f, r1, r0);
      ring_barrier(kh);
      qk = inc(qk, Q_SLOTS); ok = inc(ok, O_SLOTS);
    }
    int ent = ndiag, hh = 0;
    float beta = btab[ent < ne ? ent : 0];
#pragma unroll 1
    for (int s = nd; s < n; s += 2) {
      window_a(std::false_type{}, std::integral_constant<int, 0>{}, qring(qk), oring(ok), pbuf(0), beta, r0, r1);
      ring_barrier(kh);
      qk = inc(qk, Q_SLOTS); ok = inc(ok, O_SLOTS);
      window_a(std::false_type{}, std::integral_constant<int, 1>{}, qring(qk), oring(ok), pbuf(1), beta, r1, r0);
      ring_barrier(kh);
      qk = inc(qk, Q_SLOTS); ok = inc(ok, O_SLOTS);
      if (++hh == G) {
        hh = 0;
        ++ent;
        beta = btab[ent < ne ? ent : 0];
      }
    }
  } else {
    float gsum = 0.0f;
    int gstep = 0, gent = 0;
    float gvb = 1.0f;   // gate of the dS entry (outer; read after the first ring barrier)
    auto step_done = [&]() {
      if (++gstep < 2 * G) return;
      const float tot = wave_sum(gsum);
      gsum = 0.0f;
      gstep = 0;
      if (lane == 0) gtab[kh * kColChunkMax + gent] = tot;
      ++gent;
      if (OUTER) gvb = __builtin_amdgcn_exp2f(btab[gent < ne ? gent : 0]);
    };
    copy_next();
    copy_next();
    ring_barrier(kh);   // dO of step 0 landed (and the entry table written)
    if (OUTER) gvb = __builtin_amdgcn_exp2f(btab[0]);
    {
      const char* o0 = oring(0);
      copy_next();
      rows_product_with(o0, r0, [](int) {});   // dP_0
    }
    ring_barrier(kh);
    int ok = 1, qk = 0;
    int s = 1;
#pragma unroll 1
    for (; s + 1 < n; s += 2) {
      window_b(oring(ok), qring(qk), pbuf(0), r0, r1, gsum, gvb);   // step s - 1 is even
      ring_barrier(kh);
      step_done();
      ok = inc(ok, O_SLOTS); qk = inc(qk, Q_SLOTS);
      window_b(oring(ok), qring(qk), pbuf(1), r1, r0, gsum, gvb);
      ring_barrier(kh);
      step_done();
      ok = inc(ok, O_SLOTS); qk = inc(qk, Q_SLOTS);
    }
    window_b(oring(ok), qring(qk), pbuf(0), r0, r1, gsum, gvb);   // dP_{n-1}; dS / dK of step n - 2
    ring_barrier(kh);
    step_done();
    qk = inc(qk, Q_SLOTS);
    bf16x8 bop[2];
    {
      float dl[16];
      read_stat(qring(qk), dl);
      const _Float16* px = pbuf(1);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const f16x8 ph = *(const f16x8*)(px + (h2 * 64 + lane) * 8);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const float pj = (float)ph[x];
          const float dpj = OUTER ? r1[h2 * 8 + x] * gvb : r1[h2 * 8 + x];
          const float ds = fmaf(pj, dpj - dl[h2 * 8 + x], 0.0f);
          gsum = OUTER ? fmaf(pj, dpj, gsum) : gsum + ds;
          bop[h2][x] = (bf16)ds;
        }
      }
    }
    step_done();
    contract(qring(qk), bop, [](int) {});
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the trailing copies
  __syncthreads();   // dLogG partials of both key halves are in gtab

  // dLogG[i, j] of every entry with i != j, in its score head's gate row
  // (key halves added in order)
  if (wv == 1 && lane < ne) {
    const int code = itab[lane];
    const int ib = code / a.nsh;
    const long long bs = bhk * a.nsh + code % a.nsh;
    if (ib != j) a.dlg[(bs * a.C + ib) * a.C + j] = gtab[lane] + gtab[kColChunkMax + lane];
  }

  // epilogue: A writes dV, B writes dK (times the softmax scale), keys kh*32 + l32
  const long long orow = bhk * a.N + (long long)j * BLK + kh * 32;
  const float mul = role == 0 ? 1.0f : a.scale;
  if (only_chunk) {   // the only contributor to these rows
    bf16* dst = role == 0 ? a.dv : a.dk;
    const int key = j * BLK + kh * 32 + l32;
    if (packed && key >= sp.n) return;   // the row belongs to no sequence of this batch
    const long long r = packed ? (sp.start + key) * a.Hkv + hk : orow + l32;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 o;
#pragma unroll
        for (int y = 0; y < 4; ++y) o[y] = (bf16)(acc[dt][q4 * 4 + y] * mul);
        *(bf16x4*)(dst + r * HD + dt * 32 + q4 * 8 + g * 4) = o;
      }
  } else {
    float* dst = a.partial + (long long)gch * 2 * 8192 + (role == 0 ? 8192 : 0) + kh * 32 * HD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4*)(dst + l32 * HD + dt * 32 + q4 * 8 + g * 4) =
            f32x4{acc[dt][q4 * 4] * mul, acc[dt][q4 * 4 + 1] * mul,
                  acc[dt][q4 * 4 + 2] * mul, acc[dt][q4 * 4 + 3] * mul};
  }
}

// One workgroup per (column, quarter of its 64 x 128 tile); each lane sums
// 8 consecutive fp32 of dK and of dV over the column's chunks, in chunk order
// (deterministic), four chunks' loads in flight at a time.
__global__ void __launch_bounds__(256) reduce_kernel(BwdArgs a) {
  const long long col = blockIdx.x >> 2;   // (batch, kv head, key block)
  const int j = (int)(col % a.C);
  const long long bhk = col / a.C;
  if (a.chunkoff[col + 1] - a.chunkoff[col] <= 1) return;   // written directly
  const long long orow = bhk * a.N + (long long)j * BLK;
  const int e = (threadIdx.x + (blockIdx.x & 3) * 256) * 8;
  // packed batch: key row e / HD of the block, if it belongs to the sequence
  long long prow = -1;
  if (a.cu != nullptr) {
    const Span sp = seq_span(a, (int)(bhk / a.Hkv));
    const int key = j * BLK + e / HD;
    if (key >= sp.n) return;
    prow = (sp.start + key) * a.Hkv + (int)(bhk % a.Hkv);
  }
  f32x4 sk[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  f32x4 sv[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  const int c0 = a.chunkoff[col];
  const int nch = a.chunkoff[col + 1] - c0;
  const float* base = a.partial + (long long)c0 * 2 * 8192 + e;
  int cc = 0;
  for (; cc + 4 <= nch; cc += 4) {
    f32x4 lk[4][2], lv[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* pk = base + (long long)(cc + u) * 2 * 8192;
      lk[u][0] = *(const f32x4*)pk;
      lk[u][1] = *(const f32x4*)(pk + 4);
      lv[u][0] = *(const f32x4*)(pk + 8192);
      lv[u][1] = *(const f32x4*)(pk + 8192 + 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) { sk[h] += lk[u][h]; sv[h] += lv[u][h]; }
  }
  for (; cc < nch; ++cc) {
    const float* pk = base + (long long)cc * 2 * 8192;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sk[h] += *(const f32x4*)(pk + 4 * h);
      sv[h] += *(const f32x4*)(pk + 8192 + 4 * h);
    }
  }
  bf16x8 ok, ov;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    ok[x] = (bf16)sk[x >> 2][x & 3];
    ov[x] = (bf16)sv[x >> 2][x & 3];
  }
  const long long off = prow >= 0 ? prow * HD + e % HD : orow * HD + e;
  *(bf16x8*)(a.dk + off) = ok;
  *(bf16x8*)(a.dv + off) = ov;
}

template <int NH, bool KS = false>
hipError_t launch_dq(BwdArgs a, int head_base, int nchunk, long long units, hipStream_t st) {
  a.head_base = head_base;
  a.nchunk = nchunk;
  const dim3 grid((unsigned)(units * nchunk)), block(NH * 128 * (KS ? 2 : 1));
  const int v = (a.cu != nullptr ? 2 : 0) | (a.outer ? 1 : 0);
  switch (v) {
    case 0: hipLaunchKernelGGL((bwd_dq_kernel<NH, false, false, KS>), grid, block, 0, st, a); break;
    case 1: hipLaunchKernelGGL((bwd_dq_kernel<NH, false, true, KS>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((bwd_dq_kernel<NH, true, false, KS>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((bwd_dq_kernel<NH, true, true, KS>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace

namespace {
BwdArgs make_bwd_args(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl) {
  BwdArgs a{};
  a.q = (const bf16*)p.q; a.k = (const bf16*)p.k; a.v = (const bf16*)p.v; a.o = p.o;
  a.d_o = (const bf16*)p.d_o; a.lse = p.lse; a.lg = p.log_gate; a.sel_idx = p.sel_idx;
  a.sel_cnt = p.sel_cnt; a.dq = (bf16*)p.dq; a.dk = (bf16*)p.dk; a.dv = (bf16*)p.dv;
  a.dlg = p.dlog_gate; a.dsc = p.dscores;
  a.delta = (float*)(ws + wl.delta);
  a.lsen = (float*)(ws + wl.lsen);
  a.colmask = (uint32_t*)(ws + wl.colmask);
  a.collen = (int32_t*)(ws + wl.collen);
  a.coloff = (int32_t*)(ws + wl.coloff);
  a.chunkoff = (int32_t*)(ws + wl.chunkoff);
  a.collist = (int32_t*)(ws + wl.collist);
  a.partial = (float*)(ws + wl.partial);
  a.chunk_rank = (int32_t*)(ws + wl.chunk_rank);
  a.chunk_hist = (int32_t*)(ws + wl.chunk_hist);
  a.chunk_desc = (int32_t*)(ws + wl.chunk_desc);
  a.nrow = (long long)s.B * s.Hs * s.C;    // gate-table rows
  a.ncol = (long long)s.B * s.Hkv * s.C;   // key-major columns
  a.nsh = s.Hs / s.Hkv;
  a.Hs = s.Hs;
  a.Gs = s.Hq / s.Hs;
  a.hard = s.hard;
  a.outer = s.outer;
  a.cc = col_chunk(s);
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G; a.N = s.N; a.C = s.C; a.cap = s.cap; a.W = wl.words;
  a.o_fp32 = s.o_fp32;
  a.c2 = s.scale * kLog2e;
  a.scale = s.scale;
  a.lens = s.lens;
  a.cu = s.cu;
  a.T = s.T;
  return a;
}
}  // namespace

hipError_t launch_bwd_dq_mfma(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl,
                              hipStream_t st) {
  BwdArgs a = make_bwd_args(s, p, ws, wl);
  const long long units = (long long)s.B * s.Hkv * s.C;   // (batch, kv head, query block)
  hipError_t e;
  // column bit masks of the selection transpose: zeroed here, set by the
  // query-major kernels at the end of each gate row's work
  const long long nmask = a.ncol * a.W;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)min((nmask + 255) / 256, 65535LL)),
                     dim3(256), 0, st, a.colmask, nmask);
  // query-major pass (heads in chunks of 4, 2, 1; one head per chunk when
  // every head has its own gates and selection)
  int h = 0;
  if (a.Gs < 2 && s.G > 1) {
    e = launch_dq<1, true>(a, 0, s.G, units, st);   // one head per workgroup, keys split
    if (e != hipSuccess) return e;
    h = s.G;
  }
  if (s.G / 4 > 0 && h == 0) {
    e = launch_dq<4>(a, h, s.G / 4, units, st);
    if (e != hipSuccess) return e;
    h += 4 * (s.G / 4);
  }
  if ((s.G - h) / 2 > 0) {
    e = launch_dq<2>(a, h, 1, units, st);
    if (e != hipSuccess) return e;
    h += 2;
  }
  if (s.G - h > 0) {
    e = launch_dq<1>(a, h, 1, units, st);
    if (e != hipSuccess) return e;
  }
  // selection transpose for the key-major stage (the masks are set)
  hipLaunchKernelGGL(count_kernel, dim3((unsigned)((a.ncol + 255) / 256)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(fill_lists_kernel, dim3((unsigned)((a.ncol + 3) / 4)), dim3(256), 0, st, a);
  // schedule order of the key-major chunks
  const unsigned cgrid = (unsigned)((wl.max_chunks + 255) / 256);
  hipLaunchKernelGGL(chunk_count_kernel, dim3(cgrid), dim3(256), 0, st, a);
  hipLaunchKernelGGL(scan_ints_kernel, dim3(1), dim3(1024), 0, st, a.chunk_hist, a.ncol);
  hipLaunchKernelGGL(chunk_scatter_kernel, dim3(cgrid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_mfma(const Shape& s, const BwdPtrs& p, char* ws,
                                const BwdWorkspace& wl, hipStream_t st) {
  BwdArgs a = make_bwd_args(s, p, ws, wl);
  // dLogG: the key-major pass writes the selected entries (with hard gates
  // the dropped-block pass adds the other historical blocks of every row that
  // holds a query).  With soft gates the dScores kernel writes the rest of the
  // table as 0; otherwise it is zeroed here first.
  const bool ds_fills = p.dscores != nullptr && !s.hard;
  if (!ds_fills) {
    const long long ntab = a.nrow * s.C;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)min((ntab + 255) / 256, 65535LL)),
                       dim3(256), 0, st, (uint32_t*)a.dlg, ntab);
  }
  const dim3 kgrid((unsigned)wl.max_chunks), kblock(256);
  const int v = (s.cu != nullptr ? 2 : 0) | (s.outer ? 1 : 0);
  switch (v) {
    case 0: hipLaunchKernelGGL((bwd_dkdv_kernel<false, false>), kgrid, kblock, 0, st, a); break;
    case 1: hipLaunchKernelGGL((bwd_dkdv_kernel<false, true>), kgrid, kblock, 0, st, a); break;
    case 2: hipLaunchKernelGGL((bwd_dkdv_kernel<true, false>), kgrid, kblock, 0, st, a); break;
    default: hipLaunchKernelGGL((bwd_dkdv_kernel<true, true>), kgrid, kblock, 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long kcols = (long long)s.B * s.Hkv * s.C;   // (batch, kv head, key block)
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)(kcols * 4)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // hard gates: the gate gradients of the dropped blocks (straight-through
  // estimator); the key-major pass above wrote those of the selected blocks
  if (s.hard) {
    // dynamic LDS beside the kernel's 64 KB of tiles: the row's selection
    // bit mask and one accumulator per block (33 KB at the 8192-block limit)
    const size_t lds = ste_dynamic_lds(s.C);
    if (kSteStaticLds + lds > 160 * 1024) return hipErrorInvalidValue;   // validated on the host
    e = hipFuncSetAttribute((const void*)&ste_mfma_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(ste_mfma_kernel, dim3((unsigned)a.nrow), dim3(256), lds, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.dscores == nullptr) return hipSuccess;
  return launch_dscores(s, p.dlog_gate, p.log_gate, p.dscores, ds_fills ? p.sel_idx : nullptr,
                        p.sel_cnt, st);
}

}  // namespace sas
