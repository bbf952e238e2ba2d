// Matrix-core (MFMA) backward of SAS gated block-sparse attention, bf16
// inputs, fp32 accumulation, block b = 64, head_dim D = 128, on gfx950.
//
// Follows the recomputation backward of the SAS paper's App. E (Alg. 4):
//   Delta = rowsum(O * dO);  P = exp(S - LSE);  dS = P * (dO V^T - Delta);
//   dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO;
//   dLogG[i, m] = sum of dS over the query tokens of block i (all G heads of
//                 the kv group) and the key tokens of selected block m;
// and the selector-score gradient of App. D.3 / Eq. 8.
//
// Kernels (in launch order):
//   bwd_dq_kernel       query-major pass: one workgroup per (batch, kv head,
//                       query block, chunk of heads); each wavefront owns 64
//                       query rows of one head and streams the diagonal block
//                       and the selected blocks.  It computes Delta (from the
//                       forward output), recomputes S^T = K Q^T and
//                       dP^T = V dO^T, accumulates dQ^T += K^T dS^T in
//                       registers and reduces dS of every tile to one block
//                       log-gate gradient partial (deterministic: fixed lane
//                       butterfly, fixed wave order).
//   finalize_kernel     sums the per-head-chunk partials in a fixed order into
//                       the dense dLogG table and, optionally, applies the
//                       softmax backward to the selector scores.
//   column kernels      transpose the selection: bit (j, i) of a column mask is
//                       set when row i selected block j; each column j then
//                       gets the ascending list {j} u {i > j : j in I_i} and is
//                       cut into chunks of at most kColChunk query blocks.
//   bwd_dkdv_kernel     key-major pass: one workgroup per column chunk; K_j
//                       and V_j stay in LDS, each wavefront streams (query
//                       block, head) items, recomputes S = Q K^T and
//                       dP = dO V^T (keys in the lane dimension), and
//                       accumulates dV^T += dO^T P and dK^T += Q^T dS, with
//                       Q^T / dO^T staged transposed in wave-private LDS.  The
//                       four wavefronts' partial sums are added in a fixed order.
//   reduce_kernel       columns cut into several chunks: fp32 partials summed
//                       in chunk order (deterministic).
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
constexpr int KSTR = HD + 8;   // bf16 per row of a row-major [key][d] LDS tile
constexpr int XSTR = 32 + 4;   // bf16 per row of a wave's transposed [d][32 queries] tile

struct BwdArgs {
  const bf16* q; const bf16* k; const bf16* v; const void* o; const bf16* d_o;
  const float* lse; const float* lg; const int32_t* sel_idx; const int32_t* sel_cnt;
  bf16* dq; bf16* dk; bf16* dv; float* dlg; float* dsc;
  float* delta;
  float* dlg_part;
  uint32_t* colmask; int32_t* collen; int32_t* coloff; int32_t* chunkoff; int32_t* collist;
  float* partial;
  int32_t* chunk_rank; int32_t* chunk_hist; int32_t* chunk_order;
  long long ncol;  // B * Hkv * C (rows of the score table == columns)
  int Hq, Hkv, G, N, C, cap, W, o_fp32;
  int head_base, nchunk, part_base, nparts;
  float c2, scale;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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
// query-major pass: Delta, dQ, block log-gate gradient partials
// ---------------------------------------------------------------------------
constexpr int TILE = BLK * HD;   // bf16 elements of one 64 x 128 tile

// LDS tiles are row-major with 256-byte rows and no padding; the 16-byte chunk
// c of row r sits in slot c ^ (r & 15), so the 16 rows read by a lane group
// for one chunk land in 16 different slots (all banks).
__device__ __forceinline__ int swz(int r, int c) { return r * HD + ((c ^ (r & 15)) << 3); }

// Asynchronous global -> LDS copy of one 64 x 128 tile by NW wavefronts
// (global_load_lds_dwordx4); completion is awaited with s_waitcnt vmcnt(0).
template <int NW>
__device__ __forceinline__ void tile_to_lds(bf16* lds, const bf16* g, int w, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int r = 0; r < 16 / NW; ++r) {
    const int seg = w + NW * r;               // 1 KB segment = rows 4 seg .. 4 seg + 3
    const int row = seg * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    __builtin_amdgcn_global_load_lds(g + row * HD + c * 8, (lds_void*)(lds + seg * 512), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vm() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A column fragment (8 rows r0 + {g4*4 .. +3, 16 + g4*4 .. +3} of column
// c0 + l16) of a swizzled row-major tile, via two transposed reads.
__device__ __forceinline__ bf16x8 col_frag(const bf16* t, int r0, int c0, int l16, int g4) {
  const int r = r0 + g4 * 4 + (l16 >> 2);
  const int c = (c0 >> 3) + ((l16 >> 1) & 1);
  const int e = (c0 & 7) + (l16 & 1) * 4;
  return join(ds_read_tr(t + swz(r, c) + e), ds_read_tr(t + swz(r + 16, c) + e));
}

// One workgroup = NH query heads of one (batch, kv head, query block); two
// wavefronts per head, each owning 32 of the 64 query rows.
template <int NH>
__global__ void __launch_bounds__(NH * 128, 2) bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = 2 * NH;
  __shared__ __attribute__((aligned(16))) bf16 s_k[2][TILE];
  __shared__ __attribute__((aligned(16))) bf16 s_v[2][TILE];
  __shared__ float s_red[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int half = w & 1;

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
  float* part = a.dlg_part + ((long long)(a.part_base + chunk) * a.ncol + row) * (a.cap + 1);

  auto load_tile = [&](int kb, int stg) {
    tile_to_lds<NW>(s_k[stg], kbase + (long long)kb * TILE, w, lane);
    tile_to_lds<NW>(s_v[stg], vbase + (long long)kb * TILE, w, lane);
  };
  const int ntiles = cnt + 1;
  load_tile(i, 0);

  // Q^T and dO^T as B operands (lane: row qt*16 + l16, dims ks*32 + g4*8 .. +7)
  bf16x8 qf[2][4], dof[2][4];
  float lse2[2], dlt[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const long long r = q0 + qt * 16 + l16;
    float part_d = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int d0 = ks * 32 + g4 * 8;
      qf[qt][ks] = *(const bf16x8*)(a.q + r * HD + d0);
      dof[qt][ks] = *(const bf16x8*)(a.d_o + r * HD + d0);
      if (a.o_fp32) {
        const f32x4 o0 = *(const f32x4*)((const float*)a.o + r * HD + d0);
        const f32x4 o1 = *(const f32x4*)((const float*)a.o + r * HD + d0 + 4);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          part_d += o0[x] * (float)dof[qt][ks][x];
          part_d += o1[x] * (float)dof[qt][ks][x + 4];
        }
      } else {
        const bf16x8 ob = *(const bf16x8*)((const bf16*)a.o + r * HD + d0);
#pragma unroll
        for (int x = 0; x < 8; ++x) part_d += (float)ob[x] * (float)dof[qt][ks][x];
      }
    }
    dlt[qt] = sum4(part_d);   // Delta = rowsum(O * dO) over the 4 lanes of the row
    lse2[qt] = a.lse[r] * kLog2e;
    if (g4 == 0) a.delta[r] = dlt[qt];
  }

  f32x4 dqacc[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) dqacc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 64-key tile: recompute S^T and dP^T, form dS, accumulate dQ^T and the
  // tile's dS sum.
  auto tile = [&](auto diag_tag, int stg, float beta) -> float {
    constexpr bool DIAG = decltype(diag_tag)::value;
    const bf16* Ks = s_k[stg];
    const bf16* Vs = s_v[stg];
    float tsum = 0.0f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {   // two halves of 32 keys
      f32x4 sacc[2][2], dpacc[2][2];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          sacc[k2][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
          dpacc[k2][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int kr = (kh * 2 + k2) * 16 + l16;
          const bf16x8 ka = *(const bf16x8*)(Ks + swz(kr, ks * 4 + g4));
          const bf16x8 va = *(const bf16x8*)(Vs + swz(kr, ks * 4 + g4));
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            sacc[k2][qt] = mfma16(ka, qf[qt][ks], sacc[k2][qt]);
            dpacc[k2][qt] = mfma16(va, dof[qt][ks], dpacc[k2][qt]);
          }
        }
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float off = beta - lse2[qt];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float p = __builtin_amdgcn_exp2f(fmaf(sacc[k2][qt][j], a.c2, off));
            if (DIAG && ((kh * 2 + k2) * 16 + g4 * 4 + j > half * 32 + qt * 16 + l16)) p = 0.0f;
            const float ds = p * (dpacc[k2][qt][j] - dlt[qt]);
            if (!DIAG) tsum += ds;
            dsb[qt][k2 * 4 + j] = (bf16)ds;
          }
      }
      // dQ^T += K^T dS^T over these 32 keys (K^T fragments: transposed reads)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 ka = col_frag(Ks, kh * 32, dt * 16, l16, g4);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) dqacc[dt][qt] = mfma16(ka, dsb[qt], dqacc[dt][qt]);
      }
    }
    return tsum;
  };

  wait_vm();
  __syncthreads();
  if (ntiles > 1) load_tile(sel[0], 1);
  tile(std::true_type{}, 0, 0.0f);   // diagonal: no gate gradient
  wait_vm();
  __syncthreads();
  for (int t = 1; t < ntiles; ++t) {
    const int stg = t & 1;
    const float beta = lgrow[sel[t - 1]] * kLog2e;
    if (t + 1 < ntiles) load_tile(sel[t], stg ^ 1);
    float tsum = tile(std::false_type{}, stg, beta);
    tsum = wave_sum(tsum);
    if (lane == 0) s_red[t & 1][w] = tsum;
    // previous tile's partial (its slot was filled before the last barrier)
    if (tid == 0 && t >= 2) {
      float sum = 0.0f;
#pragma unroll
      for (int x = 0; x < NW; ++x) sum += s_red[(t - 1) & 1][x];
      part[t - 1] = sum;
    }
    wait_vm();
    __syncthreads();
  }
  if (tid == 0 && ntiles >= 2) {
    float sum = 0.0f;
#pragma unroll
    for (int x = 0; x < NW; ++x) sum += s_red[(ntiles - 1) & 1][x];
    part[ntiles - 1] = sum;
  }

  // dQ = scale * dQacc (lane: row qt*16 + l16, dims dt*16 + g4*4 .. +3)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    bf16* dp = a.dq + (q0 + qt * 16 + l16) * HD + g4 * 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      bf16x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = (bf16)(dqacc[dt][qt][j] * a.scale);
      *(bf16x4*)(dp + dt * 16) = r;
    }
  }
}

// ---------------------------------------------------------------------------
// dLogG table (sum of head-chunk partials) and optional selector-score grad
// ---------------------------------------------------------------------------
__device__ __forceinline__ int find_sel(const int32_t* sel, int cnt, int m) {
  int lo = 0, hi = cnt;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sel[mid] < m) lo = mid + 1; else hi = mid;
  }
  return (lo < cnt && sel[lo] == m) ? lo : -1;
}

__global__ void __launch_bounds__(256) finalize_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.ncol) return;
  const int i = (int)(row % a.C);
  const int cnt = min(a.sel_cnt[row], a.cap);
  const int32_t* sel = a.sel_idx + row * a.cap;
  float* drow = a.dlg + row * a.C;
  float tot = 0.0f;
  for (int m = lane; m < a.C; m += 64) {
    float val = 0.0f;
    if (m < i) {
      const int pos = find_sel(sel, cnt, m);
      if (pos >= 0) {
        for (int p = 0; p < a.nparts; ++p)
          val += a.dlg_part[((long long)p * a.ncol + row) * (a.cap + 1) + pos + 1];
      }
    }
    drow[m] = val;
    tot += val;
  }
  if (a.dsc == nullptr) return;
  tot = wave_sum(tot);
  const float* grow = a.lg + row * a.C;
  float* srow = a.dsc + row * a.C;
  for (int m = lane; m < a.C; m += 64)
    srow[m] = (m < i) ? (drow[m] - expf(grow[m]) * tot) : 0.0f;
}

// ---------------------------------------------------------------------------
// selection transpose: column lists
// ---------------------------------------------------------------------------
__global__ void fill_zero_kernel(uint32_t* p, long long n) {
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x)
    p[e] = 0u;
}

__global__ void mark_kernel(BwdArgs a) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gid / a.cap;
  const int t = (int)(gid % a.cap);
  if (row >= a.ncol) return;
  const int cnt = min(a.sel_cnt[row], a.cap);
  if (t >= cnt) return;
  const int m = a.sel_idx[row * a.cap + t];
  const int i = (int)(row % a.C);
  const long long col = row - i + m;  // same (batch, kv head), block m
  atomicOr(&a.colmask[col * a.W + (i >> 5)], 1u << (i & 31));
}

__global__ void count_kernel(BwdArgs a) {
  const long long col = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (col >= a.ncol) return;
  int L = 1;  // the diagonal block
  for (int w = 0; w < a.W; ++w) L += __popc(a.colmask[col * a.W + w]);
  a.collen[col] = L;
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
    sc += (L + kColChunk - 1) / kColChunk;
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
    oc += (L + kColChunk - 1) / kColChunk;
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
  if (lane == 0) out[0] = j;
  int run = 1;
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

// Order of the key-major work: chunks sorted by (batch, kv head, first query
// block they read).  Workgroups that run at the same time then stream nearby
// query blocks, so their Q / dO rows are shared through the L2 / MALL.  The
// order only schedules work; every result is reduced in a fixed order.
__global__ void chunk_count_kernel(BwdArgs a) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= a.chunkoff[a.ncol]) return;
  const long long col = chunk_column(a, g);
  const int c = g - a.chunkoff[col];
  const int first = a.collist[a.coloff[col] + c * kColChunk];
  const long long key = col - col % a.C + first;   // (batch, kv head) row base + first row
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

__global__ void chunk_scatter_kernel(BwdArgs a) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= a.chunkoff[a.ncol]) return;
  const long long col = chunk_column(a, g);
  const int c = g - a.chunkoff[col];
  const int first = a.collist[a.coloff[col] + c * kColChunk];
  const long long key = col - col % a.C + first;
  a.chunk_order[a.chunk_hist[key] + a.chunk_rank[g]] = g;
}

// ---------------------------------------------------------------------------
// key-major pass: dK, dV
// ---------------------------------------------------------------------------
// One workgroup per column chunk (key block j, up to kColChunk query blocks).
// Eight wavefronts = four pairs; pair `slot` streams the (query block, head)
// items slot, slot + 4, ... in two halves of 32 query rows, and the two
// wavefronts of a pair split the work by tensor:
//   wave A (role 0): S = Q K^T -> P, and dV^T += dO^T P   (dV accumulator)
//   wave B (role 1): dP = dO V^T -> dS = P (dP - Delta), dK^T += Q^T dS
// Each wavefront holds one 64 x 128 fp32 accumulator (128 registers), so two
// wavefronts fit per SIMD and every matrix product is computed once.  Per
// half item, A stages its Q rows and P in LDS, B stages its dO rows; the
// transposed operands Q^T / dO^T come from ds_read_b64_tr_b16 reads of the
// staged rows.  The four pairs advance in lockstep (two workgroup barriers
// per half item).
constexpr int KV_TILE_BYTES = BLK * KSTR * 2;                  // 17408 (padded rows)
constexpr int XH_BYTES = 32 * KSTR * 2;                          // 8704: 32 staged rows
constexpr int XP_BYTES = 32 * 64 * 4;                            // 8192: P, [value][lane]
constexpr int SLOT_BYTES = 2 * XH_BYTES + XP_BYTES;              // 25600
constexpr int DKDV_LDS = 2 * KV_TILE_BYTES + 4 * SLOT_BYTES;     // 137216
static_assert(DKDV_LDS >= 2 * 64 * 128 * 4, "reduction buffer must fit");

__global__ void __launch_bounds__(512, 2) bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[DKDV_LDS];
  bf16* Ks = (bf16*)smem;
  bf16* Vs = (bf16*)(smem + KV_TILE_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int role = w >> 2;   // 0: S / P / dV, 1: dP / dS / dK
  const int slot = w & 3;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  char* sbase = smem + 2 * KV_TILE_BYTES + slot * SLOT_BYTES;
  bf16* xq = (bf16*)sbase;                    // Q rows of the slot's half item
  bf16* xo = (bf16*)(sbase + XH_BYTES);       // dO rows
  float* xp = (float*)(sbase + 2 * XH_BYTES);  // P (fp32), [value index][lane]

  const int sid = xcd_remap(blockIdx.x, gridDim.x);
  const int total = a.chunkoff[a.ncol];
  if (sid >= total) return;
  const int g = a.chunk_order[sid];
  const long long col = chunk_column(a, g);
  const int c = g - a.chunkoff[col];
  const int nch = a.chunkoff[col + 1] - a.chunkoff[col];
  const int L = a.collen[col];
  const int e0 = c * kColChunk;
  const int e1 = min(L, e0 + kColChunk);
  const int32_t* list = a.collist + a.coloff[col];
  const int j = (int)(col % a.C);
  const long long bhk = col / a.C;
  const int hk = (int)(bhk % a.Hkv);
  const int bb = (int)(bhk / a.Hkv);

  {  // stage K_j, V_j (row-major, padded rows)
    const bf16* kt = a.k + (bhk * a.N + (long long)j * BLK) * HD;
    const bf16* vt = a.v + (bhk * a.N + (long long)j * BLK) * HD;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int cc = tid + r * 512;
      *(u32x4*)(&Ks[(cc >> 4) * KSTR + (cc & 15) * 8]) = *(const u32x4*)(kt + (cc >> 4) * HD + (cc & 15) * 8);
      *(u32x4*)(&Vs[(cc >> 4) * KSTR + (cc & 15) * 8]) = *(const u32x4*)(vt + (cc >> 4) * HD + (cc & 15) * 8);
    }
  }

  const int nitems = (e1 - e0) * a.G;
  const int myitems = slot < nitems ? (nitems - slot + 3) / 4 : 0;
  const int nsteps = 2 * myitems;            // this pair's half items
  const int lockstep = 2 * ((nitems + 3) / 4);   // half items of the busiest pair

  // first query row of half item s of this pair
  auto step_row0 = [&](int s) -> long long {
    const int it = slot + 4 * (s >> 1);
    const int i = list[e0 + it / a.G];
    const int h = hk * a.G + it % a.G;
    return ((long long)bb * a.Hq + h) * a.N + (long long)i * BLK + (s & 1) * 32;
  };
  // A loads Q rows, B loads dO rows (lane: row q2*16 + l16, dims ks*32 + g4*8 .. +7)
  const bf16* src = role == 0 ? a.q : a.d_o;
  auto load_rows = [&](int s, bf16x8 (&rw)[2][4]) {
    const long long r0 = step_row0(s);
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        rw[q2][ks] = *(const bf16x8*)(src + (r0 + q2 * 16 + l16) * HD + ks * 32 + g4 * 8);
  };
  // A: LSE (log2 units folded later), B: Delta, of this lane's accumulator rows
  const float* stat = role == 0 ? a.lse : a.delta;

  f32x4 acc[8][4];   // A: dV^T, B: dK^T  (lane: key kt*16 + l16, dims dt*16 + g4*4 .. +3)
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc[dt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 rows[2][4];
  if (nsteps > 0) load_rows(0, rows);
  __syncthreads();   // K_j, V_j staged

#pragma unroll 1
  for (int s = 0; s < lockstep; ++s) {
    const bool active = s < nsteps;
    bf16x8 bop[4];   // B operand of this wave's accumulation (A: P, B: dS)
    f32x4 sacc[2][4];
    f32x4 st[2];
    bool diag = false;
    int hq = s & 1;
    if (active) {
      const int it = slot + 4 * (s >> 1);
      const int i = list[e0 + it / a.G];
      diag = (i == j);
      const long long r0 = step_row0(s);
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) st[q2] = *(const f32x4*)(stat + r0 + q2 * 16 + g4 * 4);
      // stage the rows for the partner's transposed reads
      bf16* xs = role == 0 ? xq : xo;
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          *(bf16x8*)(xs + (q2 * 16 + l16) * KSTR + ks * 32 + g4 * 8) = rows[q2][ks];
      // A: S = Q K^T   B: dP = dO V^T   (lane: key kt*16 + l16; rows q2*16 + g4*4 + jj)
      const bf16* T = role == 0 ? Ks : Vs;
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sacc[q2][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8 tb = *(const bf16x8*)(T + (kt * 16 + l16) * KSTR + ks * 32 + g4 * 8);
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2) sacc[q2][kt] = mfma16(rows[q2][ks], tb, sacc[q2][kt]);
        }
      if (role == 0) {
        // P = exp2(c2 s + beta - lse2): kept as bf16 B operand (dV) and as
        // fp32 in LDS for the partner's dS
        const float beta = diag ? 0.0f : a.lg[(bhk * a.C + i) * a.C + j] * kLog2e;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              float p = __builtin_amdgcn_exp2f(
                  fmaf(sacc[q2][kt][jj], a.c2, fmaf(-st[q2][jj], kLog2e, beta)));
              if (diag && (kt * 16 + l16) > (hq * 32 + q2 * 16 + g4 * 4 + jj)) p = 0.0f;
              bop[kt][q2 * 4 + jj] = (bf16)p;
              xp[((kt * 2 + q2) * 4 + jj) * 64 + lane] = p;
            }
      }
      if (s + 1 < nsteps) load_rows(s + 1, rows);
    }
    __syncthreads();   // staged rows and P visible to the partner
    if (active) {
      if (role == 1) {
        // dS = P (dP - Delta), as the B operand of dK^T += Q^T dS
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int q2 = 0; q2 < 2; ++q2)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const float p = xp[((kt * 2 + q2) * 4 + jj) * 64 + lane];
              bop[kt][q2 * 4 + jj] = (bf16)(p * (sacc[q2][kt][jj] - st[q2][jj]));
            }
      }
      // A: dV^T += dO^T P   B: dK^T += Q^T dS  (A operands: transposed reads of
      // the partner's staged rows: lane gets 4 consecutive rows of its column)
      const bf16* xt = role == 0 ? xo : xq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int ro = (g4 * 4 + (l16 >> 2)) * KSTR + dt * 16 + (l16 & 3) * 4;
        const bf16x8 ta = join(ds_read_tr(xt + ro), ds_read_tr(xt + ro + 16 * KSTR));
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[dt][kt] = mfma16(ta, bop[kt], acc[dt][kt]);
      }
    }
    __syncthreads();   // the slot's buffers are free for the next half item
  }

  // add the four pairs' partial sums in a fixed order (LDS, fp32); the 16-byte
  // chunk c of key row r is stored at chunk c ^ (r & 31) so that the 16 rows
  // written by one instruction spread over the banks
  float* redv = (float*)smem;      // role 0 accumulates dV
  float* redk = redv + 64 * 128;   // role 1 accumulates dK
  float* red = role == 0 ? redv : redk;
  auto roff = [](int r, int d) { return r * 128 + ((((d >> 2) ^ (r & 31))) << 2) + (d & 3); };
  for (int x = 0; x < 4; ++x) {
    if (slot == x) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int off = roff(kt * 16 + l16, dt * 16 + g4 * 4);
          if (x == 0) *(f32x4*)(red + off) = acc[dt][kt];
          else *(f32x4*)(red + off) += acc[dt][kt];
        }
    }
    __syncthreads();
  }
  const long long orow = bhk * a.N + (long long)j * BLK;
  if (nch == 1) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int e = (tid + r * 512) * 8;   // 8 consecutive elements of key row e / 128
      const int kr = e >> 7, d = e & 127;
      const f32x4 k0 = *(const f32x4*)(redk + roff(kr, d));
      const f32x4 k1 = *(const f32x4*)(redk + roff(kr, d + 4));
      const f32x4 v0 = *(const f32x4*)(redv + roff(kr, d));
      const f32x4 v1 = *(const f32x4*)(redv + roff(kr, d + 4));
      bf16x8 ok, ov;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        ok[x] = (bf16)(k0[x] * a.scale);
        ok[x + 4] = (bf16)(k1[x] * a.scale);
        ov[x] = (bf16)v0[x];
        ov[x + 4] = (bf16)v1[x];
      }
      *(bf16x8*)(a.dk + orow * HD + e) = ok;
      *(bf16x8*)(a.dv + orow * HD + e) = ov;
    }
  } else {
    float* pk = a.partial + (long long)g * 2 * 8192;
    float* pv = pk + 8192;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = (tid + r * 512) * 4;
      const int kr = e >> 7, d = e & 127;
      *(f32x4*)(pk + e) = *(const f32x4*)(redk + roff(kr, d));
      *(f32x4*)(pv + e) = *(const f32x4*)(redv + roff(kr, d));
    }
  }
}

__global__ void __launch_bounds__(256) reduce_kernel(BwdArgs a) {
  const long long col = blockIdx.x;
  const int c0 = a.chunkoff[col];
  const int nch = a.chunkoff[col + 1] - c0;
  if (nch <= 1) return;
  const int j = (int)(col % a.C);
  const long long bhk = col / a.C;
  const long long orow = bhk * a.N + (long long)j * BLK;
  for (int r = 0; r < 4; ++r) {
    const int e = (threadIdx.x + r * 256) * 8;
    float sk[8], sv[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) { sk[x] = 0.0f; sv[x] = 0.0f; }
    for (int cc = 0; cc < nch; ++cc) {
      const float* pk = a.partial + (long long)(c0 + cc) * 2 * 8192 + e;
      const float* pv = pk + 8192;
#pragma unroll
      for (int x = 0; x < 8; ++x) { sk[x] += pk[x]; sv[x] += pv[x]; }
    }
    bf16x8 ok, ov;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      ok[x] = (bf16)(sk[x] * a.scale);
      ov[x] = (bf16)sv[x];
    }
    *(bf16x8*)(a.dk + orow * HD + e) = ok;
    *(bf16x8*)(a.dv + orow * HD + e) = ov;
  }
}

template <int NH>
hipError_t launch_dq(BwdArgs a, int head_base, int nchunk, int part_base, long long units,
                     hipStream_t st) {
  a.head_base = head_base;
  a.nchunk = nchunk;
  a.part_base = part_base;
  hipLaunchKernelGGL((bwd_dq_kernel<NH>), dim3((unsigned)(units * nchunk)), dim3(NH * 128), 0, st,
                     a);
  return hipGetLastError();
}

}  // namespace

int bwd_head_parts(int G) { return G / 4 + (G % 4) / 2 + (G % 2); }

namespace {
BwdArgs make_bwd_args(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl) {
  BwdArgs a{};
  a.q = (const bf16*)p.q; a.k = (const bf16*)p.k; a.v = (const bf16*)p.v; a.o = p.o;
  a.d_o = (const bf16*)p.d_o; a.lse = p.lse; a.lg = p.log_gate; a.sel_idx = p.sel_idx;
  a.sel_cnt = p.sel_cnt; a.dq = (bf16*)p.dq; a.dk = (bf16*)p.dk; a.dv = (bf16*)p.dv;
  a.dlg = p.dlog_gate; a.dsc = p.dscores;
  a.delta = (float*)(ws + wl.delta);
  a.dlg_part = (float*)(ws + wl.dlg_part);
  a.colmask = (uint32_t*)(ws + wl.colmask);
  a.collen = (int32_t*)(ws + wl.collen);
  a.coloff = (int32_t*)(ws + wl.coloff);
  a.chunkoff = (int32_t*)(ws + wl.chunkoff);
  a.collist = (int32_t*)(ws + wl.collist);
  a.partial = (float*)(ws + wl.partial);
  a.chunk_rank = (int32_t*)(ws + wl.chunk_rank);
  a.chunk_hist = (int32_t*)(ws + wl.chunk_hist);
  a.chunk_order = (int32_t*)(ws + wl.chunk_order);
  a.ncol = (long long)s.B * s.Hkv * s.C;
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G; a.N = s.N; a.C = s.C; a.cap = s.cap; a.W = wl.words;
  a.o_fp32 = s.o_fp32;
  a.nparts = bwd_head_parts(s.G);
  a.c2 = s.scale * kLog2e;
  a.scale = s.scale;
  return a;
}
}  // namespace

hipError_t launch_bwd_dq_mfma(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl,
                              hipStream_t st) {
  BwdArgs a = make_bwd_args(s, p, ws, wl);
  const long long units = a.ncol;
  hipError_t e;
  // query-major pass (heads in chunks of 4, 2, 1)
  int h = 0, part = 0;
  if (s.G / 4 > 0) {
    e = launch_dq<4>(a, h, s.G / 4, part, units, st);
    if (e != hipSuccess) return e;
    part += s.G / 4;
    h += 4 * (s.G / 4);
  }
  if ((s.G - h) / 2 > 0) {
    e = launch_dq<2>(a, h, 1, part, units, st);
    if (e != hipSuccess) return e;
    part += 1;
    h += 2;
  }
  if (s.G - h > 0) {
    e = launch_dq<1>(a, h, 1, part, units, st);
    if (e != hipSuccess) return e;
  }
  // dLogG table and selector-score gradient
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((a.ncol + 3) / 4)), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // selection transpose for the key-major stage
  const long long nmask = a.ncol * a.W;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)min((nmask + 255) / 256, 65535LL)),
                     dim3(256), 0, st, a.colmask, nmask);
  const long long nmark = a.ncol * s.cap;
  hipLaunchKernelGGL(mark_kernel, dim3((unsigned)((nmark + 255) / 256)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(count_kernel, dim3((unsigned)((a.ncol + 255) / 256)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, a);
  hipLaunchKernelGGL(fill_lists_kernel, dim3((unsigned)((a.ncol + 3) / 4)), dim3(256), 0, st, a);
  // schedule order of the key-major chunks
  const unsigned cgrid = (unsigned)((wl.max_chunks + 255) / 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)min((a.ncol + 256) / 256, 65535LL)),
                     dim3(256), 0, st, (uint32_t*)a.chunk_hist, a.ncol + 1);
  hipLaunchKernelGGL(chunk_count_kernel, dim3(cgrid), dim3(256), 0, st, a);
  hipLaunchKernelGGL(scan_ints_kernel, dim3(1), dim3(1024), 0, st, a.chunk_hist, a.ncol);
  hipLaunchKernelGGL(chunk_scatter_kernel, dim3(cgrid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_mfma(const Shape& s, const BwdPtrs& p, char* ws,
                                const BwdWorkspace& wl, hipStream_t st) {
  BwdArgs a = make_bwd_args(s, p, ws, wl);
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)wl.max_chunks), dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)a.ncol), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sas
