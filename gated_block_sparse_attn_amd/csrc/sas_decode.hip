// Sparse decode: one new query token per sequence attends its current block
// and the Top-K blocks chosen from the selector scores, gathered from a paged
// KV cache.
//
// SAS paper (arXiv 2609.13141): Sec. 4.3 Alg. 2 (inference step: I =
// Top-K(s, K), S = B0 u U_{m in I} B_m, o = softmax(q K_S^T) V_S, no gates);
// Sec. 5.1 "Inference implementation" (per-query-group selection with GQA,
// only the selected KV blocks are gathered from the paged cache, batched
// decoding); Sec. 6.3 / Fig. 7(c) (Top-K ranking dominates the step at long
// context, so the selection gets a workgroup per row).
//
// Kernels:
//   decode_select_kernel   one workgroup per (sequence, kv head): stages the
//                          row's historical scores as order-preserving
//                          integer keys in LDS, finds the K-th largest key by
//                          four 8-bit MSB-first radix passes (LDS histogram +
//                          one wavefront's suffix scan), then compacts
//                          {m : key >= tau} in ascending order.
//   decode_attn_kernel     one workgroup per (sequence, kv head, tile): tile
//                          0 is the current block (tokens up to the query),
//                          tile t >= 1 the (t-1)-th selected block.  The K / V
//                          block is read once from its page (shared by the G
//                          query heads of the group), scores and the tile's
//                          softmax statistics go to a workspace partial.
//   decode_combine_kernel  one wavefront per (sequence, query head): merges
//                          the partials in tile order (deterministic).
// All three are memory-bound: HBM bytes are the selected K / V blocks.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "../../include/sas.h"
#include "sas_internal.h"

namespace sas {
namespace {

__device__ __forceinline__ uint32_t f2key(float x) {
  const uint32_t b = __float_as_uint(x);
  return b ^ ((b >> 31) ? 0xFFFFFFFFu : 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float(k ^ ((k >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}
__device__ __forceinline__ int rank_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Current block of a sequence of n tokens (query at position n - 1), with n
// clamped into [1, cmax * blk]; *bad is set when n was out of range.
__device__ __forceinline__ int current_block(int n, int blk, int cmax, int* nn, bool* bad) {
  int v = n;
  if (v < 1 || v > cmax * blk) {
    *bad = true;
    v = v < 1 ? 1 : cmax * blk;
  }
  *nn = v;
  return (v - 1) / blk;
}

constexpr int kSelMaxThreads = 1024;   // 256 for rows under 512 blocks, 1024 otherwise

__global__ void __launch_bounds__(kSelMaxThreads) decode_select_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
    float* __restrict__ tau, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
    int32_t* __restrict__ d_status, int Hkv, int cmax, int blk, int K, int cap) {
  extern __shared__ uint32_t s_key[];          // cmax keys
  __shared__ int s_hist[256];
  __shared__ int s_wave[kSelMaxThreads / 64];
  __shared__ uint32_t s_pick[2];               // digit, count above it
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const long long row = blockIdx.x;            // b * Hkv + h
  const int b = (int)(row / Hkv);
  int n;
  bool bad = false;
  const int c = current_block(seq_lens[b], blk, cmax, &n, &bad);
  const float* srow = scores + row * (long long)cmax;
  for (int m = tid; m < c; m += nthr) s_key[m] = f2key(srow[m] + 0.0f);   // -0 -> +0
  __syncthreads();

  uint32_t tkey;   // select m iff key >= tkey; none when K == 0
  bool none = false;
  if (K >= c) {
    tkey = 0u;
  } else if (K == 0) {
    tkey = 0xFFFFFFFFu;
    none = true;
  } else {
    uint32_t prefix = 0u, mask = 0u;
    int kk = K;   // rank of the wanted key among the keys matching prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int x = tid; x < 256; x += nthr) s_hist[x] = 0;
      __syncthreads();
      // histogram of the next digit over the keys matching the prefix; the
      // wave's most common case -- every candidate with the first
      // candidate's digit -- is one atomic (scores of one row share their
      // leading bits, which would otherwise serialise on one bin)
      for (int m0 = 0; m0 < c; m0 += nthr) {
        const int m = m0 + tid;
        const uint32_t k = m < c ? s_key[m] : 0u;
        const bool cand = m < c && (k & mask) == prefix;
        const uint32_t dg = (k >> shift) & 255u;
        const unsigned long long cb = __ballot(cand);
        if (cb != 0ull) {
          const int first = __builtin_ctzll(cb);
          const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)dg, first);
          const bool same = cand && dg == d0;
          const unsigned long long sb = __ballot(same);
          if (lane == first) atomicAdd(&s_hist[d0], __popcll(sb));
          if (cand && !same) atomicAdd(&s_hist[dg], 1);
        }
      }
      __syncthreads();
      if (w == 0) {
        // lane l holds digits 255 - 4l .. 252 - 4l (descending); inclusive
        // prefix over lanes = keys with a digit >= 252 - 4l
        int v4[4], v = 0;
#pragma unroll
        for (int x = 0; x < 4; ++x) { v4[x] = s_hist[255 - 4 * lane - x]; v += v4[x]; }
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (lane >= o) incl += y;
        }
        const unsigned long long hit = __ballot(incl >= kk);
        const int L = __builtin_ctzll(hit);   // kk <= #candidates, so some lane hits
        if (lane == L) {
          int cum = incl - v;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            if (cum + v4[x] >= kk) {
              s_pick[0] = (uint32_t)(255 - 4 * lane - x);
              s_pick[1] = (uint32_t)cum;
              break;
            }
            cum += v4[x];
          }
        }
      }
      __syncthreads();
      prefix |= s_pick[0] << shift;
      mask |= 255u << shift;
      kk -= (int)s_pick[1];
      __syncthreads();
    }
    tkey = prefix;
  }

  // ascending compaction of {m < c : key_m >= tkey}
  int32_t* out = sel_idx + row * (long long)cap;
  int base = 0;
  for (int m0 = 0; m0 < c; m0 += nthr) {
    const int m = m0 + tid;
    const bool p = !none && m < c && s_key[m] >= tkey;
    const unsigned long long bits = __ballot(p);
    if (lane == 0) s_wave[w] = __popcll(bits);
    __syncthreads();
    int off = base;
    for (int x = 0; x < w; ++x) off += s_wave[x];
    if (p) {
      const int pos = off + rank_below(bits);
      if (pos < cap) out[pos] = m;
    }
    for (int x = 0; x < nthr / 64; ++x) base += s_wave[x];
    __syncthreads();
  }
  for (int pos = base + tid; pos < cap; pos += nthr) out[pos] = -1;
  if (tid == 0) {
    sel_cnt[row] = base;
    if (tau != nullptr) tau[row] = (K >= c) ? -INFINITY : (none ? INFINITY : key2f(tkey));
    if (d_status != nullptr) {
      if (bad) *d_status = SAS_E_INVALID;
      else if (base > cap) *d_status = SAS_E_CAPACITY;
    }
  }
}

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return (float)(*p); }

// 16-byte chunk of T values -> float
template <typename T> struct Chunk;
template <> struct Chunk<__bf16> {
  static constexpr int N = 8;
  __device__ static void get(const uint4& u, float* f) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const bf16x8 v = __builtin_bit_cast(bf16x8, u);
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = (float)v[x];
  }
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void get(const uint4& u, float* f) {
    const float4 v = __builtin_bit_cast(float4, u);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
};
// two consecutive T values -> float
__device__ __forceinline__ float2 get2(const __bf16* p) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = *(const bf16x2*)p;
  return make_float2((float)v[0], (float)v[1]);
}
__device__ __forceinline__ float2 get2(const float* p) { return *(const float2*)p; }

struct DecArgs {
  const void* q; const void* kp; const void* vp; const int32_t* bt; const int32_t* seq_lens;
  const int32_t* sel_idx; const int32_t* sel_cnt; void* o; float* lse; float* part;
  int32_t* d_status;
  int Hq, Hkv, G, cmax, pool, cap, T;
  float c2;   // sm_scale * log2(e)
};

constexpr int kAttnThreads = 256;

// LDS bytes of one decode_attn_kernel workgroup: K and V blocks in the input
// type, the G scaled queries and the G x BLK probabilities in fp32.
template <typename T, int D, int BLK>
constexpr size_t attn_lds(int G) {
  return 2 * (size_t)BLK * D * sizeof(T) + sizeof(float) * ((size_t)G * D + (size_t)G * BLK);
}

template <typename T, int D, int BLK>
__global__ void __launch_bounds__(kAttnThreads) decode_attn_kernel(DecArgs a) {
  constexpr int EPC = Chunk<T>::N;       // elements per 16-byte chunk
  constexpr int NCH = D / EPC;           // chunks per row
  constexpr int SWM = NCH < 16 ? NCH - 1 : 15;
  extern __shared__ uint4 smem4[];
  uint4* ks = smem4;                     // BLK x NCH chunks; chunk c of row r at c ^ (r & SWM)
  uint4* vs = ks + BLK * NCH;            // BLK x NCH chunks, row-major
  float* qs = (float*)(vs + BLK * NCH);  // G x D, pre-scaled by c2
  float* ps = qs + a.G * D;              // G x BLK
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;             // b * Hkv + hk
  const int t = blockIdx.y;              // 0: current block, t >= 1: selected entry t - 1
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.G;
  int n;
  bool bad = false;
  const int c = current_block(a.seq_lens[b], BLK, a.cmax, &n, &bad);
  const int cnt = min(max(a.sel_cnt[bh], 0), a.cap);
  float* part = a.part + ((long long)bh * a.T + t) * G * (D + 2);

  int blkid = c, nkeys = n - c * BLK;
  if (t > 0) {
    if (t > cnt) {   // no such tile: empty partial
      for (int hh = tid; hh < G; hh += kAttnThreads) {
        part[hh * (D + 2) + D] = -INFINITY;
        part[hh * (D + 2) + D + 1] = 0.0f;
      }
      return;
    }
    blkid = a.sel_idx[(long long)bh * a.cap + t - 1];
    nkeys = BLK;
    if (blkid < 0 || blkid >= c) {   // not a historical block: flag, attend nothing
      bad = true;
      nkeys = 0;
      blkid = 0;
    }
  }
  int page = a.bt[(long long)b * a.cmax + blkid];
  if (page < 0 || page >= a.pool) {
    bad = true;
    page = 0;
    nkeys = 0;
  }
  if (bad && tid == 0 && a.d_status != nullptr) *a.d_status = SAS_E_INVALID;

  // stage the K / V block (16-byte chunks) and the scaled queries
  const uint4* kg = (const uint4*)((const T*)a.kp + (((long long)page * a.Hkv + hk) * BLK) * D);
  const uint4* vg = (const uint4*)((const T*)a.vp + (((long long)page * a.Hkv + hk) * BLK) * D);
  constexpr int TOTAL = BLK * NCH;
  constexpr bool EVEN = TOTAL % kAttnThreads == 0;
  constexpr int PER = (TOTAL + kAttnThreads - 1) / kAttnThreads;   // chunks per thread
  uint4 kr[PER], vr[PER];
#pragma unroll
  for (int x = 0; x < PER; ++x) {   // every load issued before the first LDS store
    const int ch = tid + x * kAttnThreads;
    kr[x] = make_uint4(0u, 0u, 0u, 0u);
    vr[x] = kr[x];
    if (EVEN || ch < TOTAL) {
      kr[x] = kg[ch];
      vr[x] = vg[ch];
    }
  }
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    const int ch = tid + x * kAttnThreads;
    if (EVEN || ch < TOTAL) {
      const int r = ch / NCH, cc = ch % NCH;
      ks[r * NCH + (cc ^ (r & SWM))] = kr[x];
      vs[ch] = vr[x];
    }
  }
  const T* qg = (const T*)a.q + ((long long)b * a.Hq + hk * G) * D;
  for (int e = tid; e < G * D; e += kAttnThreads) qs[e] = ld(qg + e) * a.c2;
  __syncthreads();

  // scores (log2 units) and the tile's softmax statistics: pair (hh, kk),
  // kk fastest, so each head's BLK keys are one aligned segment of a wavefront
  for (int pr0 = 0; pr0 < G * BLK; pr0 += kAttnThreads) {
    const int pr = pr0 + tid;
    const int hh = pr / BLK, kk = pr % BLK;
    float z = -INFINITY;
    if (hh < G && kk < nkeys) {
      float acc = 0.0f;
#pragma unroll 4
      for (int cc = 0; cc < NCH; ++cc) {
        float kf[EPC];
        Chunk<T>::get(ks[kk * NCH + (cc ^ (kk & SWM))], kf);
        const float* qp = qs + hh * D + cc * EPC;
#pragma unroll
        for (int x = 0; x < EPC; ++x) acc = fmaf(qp[x], kf[x], acc);
      }
      z = acc;
    }
    float mx = z;
#pragma unroll
    for (int o = BLK / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    const float p = (mx == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(z - mx);
    float l = p;
#pragma unroll
    for (int o = BLK / 2; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    if (hh < G) {
      ps[hh * BLK + kk] = p;
      if (kk == 0) {
        part[hh * (D + 2) + D] = mx;
        part[hh * (D + 2) + D + 1] = l;
      }
    }
  }
  __syncthreads();

  // unnormalised output of the tile: acc[hh][d] = sum_kk p[hh][kk] v[kk][d]
  const T* vrow = (const T*)vs;
  for (int e = tid; e < G * (D / 2); e += kAttnThreads) {
    const int hh = e / (D / 2), d = (e % (D / 2)) * 2;
    float o0 = 0.0f, o1 = 0.0f;
    for (int kk = 0; kk < nkeys; ++kk) {
      const float p = ps[hh * BLK + kk];
      const float2 v2 = get2(vrow + kk * D + d);
      o0 = fmaf(p, v2.x, o0);
      o1 = fmaf(p, v2.y, o1);
    }
    part[hh * (D + 2) + d] = o0;
    part[hh * (D + 2) + d + 1] = o1;
  }
}

// ---- matrix-core tile kernel (bf16, D = 128, b = 64, G <= 32) ----
// One wavefront per (sequence, kv head, tile), the same partials as
// decode_attn_kernel.  The G query heads are the columns of two 32x32x16
// MFMA products: S^T = K Q^T (A: key rows of the block, read straight from
// the page; B: the heads' queries, columns >= G zero) and O^T = V^T P^T (A:
// transposed reads of the V block staged in LDS; B: the bf16 probabilities,
// whose accumulator layout already is the B operand's).  Each head's 64
// scores sit in one column, i.e. in lanes h and h + 32.
typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 dbf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 dbf16x2 __attribute__((ext_vector_type(2)));
typedef float df32x16 __attribute__((ext_vector_type(16)));
typedef float df32x4 __attribute__((ext_vector_type(4)));
typedef float df32x2 __attribute__((ext_vector_type(2)));
constexpr int kMD = 128, kMB = 64;

// element offset of 16-byte chunk c of row r in the staged V block
__device__ __forceinline__ int dswz(int r, int c) { return r * kMD + ((c ^ slot16(r)) << 3); }
// gfx950 transposed LDS read: within each 16-lane group, lane u gets element
// u % 4 of the 8-byte chunks addressed by lanes u / 4 + 4x (x = 0..3)
__device__ __forceinline__ dbf16x4 dread_tr(const __bf16* p) {
  typedef __attribute__((address_space(3))) dbf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}
// v_mfma_f32_32x32x16_bf16: lane l (g = l / 32): A row l % 32, k = 8 g .. +7;
// B column l % 32, same k; C column l % 32, rows 8 (jj / 4) + 4 g + jj % 4
__device__ __forceinline__ df32x16 dmfma(dbf16x8 a, dbf16x8 b, df32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// max / sum over the lanes l and l ^ 32 (the two lanes of a C column)
__device__ __forceinline__ float dmax2(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float dsum2(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ void __launch_bounds__(64) decode_attn_mfma_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 vs[kMB * kMD];
  const int lane = threadIdx.x;
  const int g = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x;             // b * Hkv + hk
  const int t = blockIdx.y;              // 0: current block, t >= 1: selected entry t - 1
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.G;
  int n;
  bool bad = false;
  const int c = current_block(a.seq_lens[b], kMB, a.cmax, &n, &bad);
  const int cnt = min(max(a.sel_cnt[bh], 0), a.cap);
  float* part = a.part + ((long long)bh * a.T + t) * G * (kMD + 2);

  int blkid = c, nkeys = n - c * kMB;
  if (t > 0) {
    if (t > cnt) {   // no such tile: empty partial
      if (lane < G) {
        part[lane * (kMD + 2) + kMD] = -INFINITY;
        part[lane * (kMD + 2) + kMD + 1] = 0.0f;
      }
      return;
    }
    blkid = a.sel_idx[(long long)bh * a.cap + t - 1];
    nkeys = kMB;
    if (blkid < 0 || blkid >= c) {   // not a historical block: flag, attend nothing
      bad = true;
      nkeys = 0;
      blkid = 0;
    }
  }
  int page = a.bt[(long long)b * a.cmax + blkid];
  if (page < 0 || page >= a.pool) {
    bad = true;
    page = 0;
    nkeys = 0;
  }
  if (bad && lane == 0 && a.d_status != nullptr) *a.d_status = SAS_E_INVALID;

  const __bf16* kg = (const __bf16*)a.kp + (((long long)page * a.Hkv + hk) * kMB) * kMD;
  const __bf16* vg = (const __bf16*)a.vp + (((long long)page * a.Hkv + hk) * kMB) * kMD;
  // V block -> LDS: 16 asynchronous copies of 1 KB (rows 4 s .. 4 s + 3), each
  // lane fetching the chunk that its LDS slot holds under the swizzle
#pragma unroll
  for (int sg = 0; sg < 16; ++sg) {
    const int row = sg * 4 + (lane >> 4);
    const int ch = (lane & 15) ^ slot16(row);
    dma16(vg + row * kMD + ch * 8, lds_addr(vs + sg * 512));
  }
  // K rows (A operand): key kh * 32 + l32, dims ks * 16 + 8 g .. +7
  dbf16x8 ka[2][8];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      ka[kh][ks] = *(const dbf16x8*)(kg + (kh * 32 + l32) * kMD + ks * 16 + g * 8);
  // queries (B operand): head l32 of the group, dims ks * 16 + 8 g .. +7
  dbf16x8 qf[8];
  const __bf16* qg = (const __bf16*)a.q + ((long long)b * a.Hq + hk * G + min(l32, G - 1)) * kMD;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qf[ks] = *(const dbf16x8*)(qg + ks * 16 + g * 8);
    if (l32 >= G) qf[ks] = dbf16x8{};
  }
  // S^T of the two 32-key halves
  df32x16 sc[2];
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    sc[kh] = df32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sc[kh] = dmfma(ka[kh][ks], qf[ks], sc[kh]);
  }
  // the head's softmax statistics over the tile (log2 units; keys past the
  // query are masked)
  float mx = -INFINITY;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int key = kh * 32 + 8 * (jj >> 2) + 4 * g + (jj & 3);
      const float z = key < nkeys ? sc[kh][jj] * a.c2 : -INFINITY;
      sc[kh][jj] = z;
      mx = fmaxf(mx, z);
    }
  mx = dmax2(mx);
  float l = 0.0f;
  dbf16x8 pb[2][2];   // [half][16-key slice]: B operand of O^T
#pragma unroll
  for (int kh = 0; kh < 2; ++kh)
#pragma unroll
    for (int jj = 0; jj < 16; jj += 2) {
      df32x2 pp;
      pp[0] = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[kh][jj] - mx);
      pp[1] = mx == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[kh][jj + 1] - mx);
      l += pp[0] + pp[1];
      const dbf16x2 h2 = __builtin_convertvector(pp, dbf16x2);
      pb[kh][jj >> 3][jj & 7] = h2[0];
      pb[kh][jj >> 3][(jj & 7) + 1] = h2[1];
    }
  l = dsum2(l);
  // O^T = V^T P^T: head-dim tiles dt, A fragments (dims dt * 32 + l32, keys
  // 16 sl + {4 g .. 4 g + 3, 8 + 4 g .. 8 + 4 g + 3}) by transposed reads
  const int u = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the V copies (and loads) landed
  __syncthreads();
  df32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    oacc[dt] = df32x16{};
    const int o0 = dswz(g * 4 + (u >> 2), dt * 4 + dhalf * 2 + ((u >> 1) & 1)) + (u & 1) * 4;
    const int o1 = dswz(g * 4 + (u >> 2) + 8, dt * 4 + dhalf * 2 + ((u >> 1) & 1)) + (u & 1) * 4;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const __bf16* vp = vs + (kh * 32 + sl * 16) * kMD;
        const dbf16x8 va = __builtin_shufflevector(dread_tr(vp + o0), dread_tr(vp + o1),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
        oacc[dt] = dmfma(va, pb[kh][sl], oacc[dt]);
      }
  }
  // partial of head l32: unnormalised output (dims dt * 32 + 8 q4 + 4 g .. +3), max, sum
  if (l32 < G) {
    float* ph = part + l32 * (kMD + 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int y = 0; y < 4; ++y) ph[dt * 32 + q4 * 8 + g * 4 + y] = oacc[dt][q4 * 4 + y];
    if (g == 0) {
      ph[kMD] = mx;
      ph[kMD + 1] = l;
    }
  }
}

// merge the tile partials of one (sequence, query head): wavefront w takes
// tiles w, w + 4, ... (lane t of a 64-tile chunk reads a tile's (m, l); the
// output rows are streamed with independent loads, the tile's scale coming
// by readlane); the four wavefronts are then added in a fixed order.
constexpr int kCombWaves = 4;

template <typename T, int D>
__global__ void __launch_bounds__(64 * kCombWaves) decode_combine_kernel(DecArgs a) {
  __shared__ float s_red[kCombWaves][D + 2];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int bq = blockIdx.x;                  // b * Hq + h
  const int b = bq / a.Hq, h = bq % a.Hq;
  const int hk = h / a.G, hh = h % a.G;
  const int bh = b * a.Hkv + hk;
  const int nt = min(max(a.sel_cnt[bh], 0), a.cap) + 1;
  const float* p0 = a.part + (long long)bh * a.T * a.G * (D + 2) + hh * (D + 2);
  const long long stride = (long long)a.G * (D + 2);
  float M = -INFINITY;
  for (int t = threadIdx.x; t < nt; t += 64 * kCombWaves) M = fmaxf(M, p0[t * stride + D]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if (lane == 0) s_red[w][0] = M;
  __syncthreads();
  M = s_red[0][0];
#pragma unroll
  for (int x = 1; x < kCombWaves; ++x) M = fmaxf(M, s_red[x][0]);
  __syncthreads();
  float L = 0.0f;
  float acc[D / 64];
#pragma unroll
  for (int x = 0; x < D / 64; ++x) acc[x] = 0.0f;
  // this wavefront's tiles: w + kCombWaves * j
  const int nw = nt > w ? (nt - w + kCombWaves - 1) / kCombWaves : 0;
  for (int j0 = 0; j0 < nw; j0 += 64) {
    const int t = w + kCombWaves * (j0 + lane);
    float sc = 0.0f;
    if (j0 + lane < nw) {
      const float m = p0[t * stride + D];
      sc = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      L = fmaf(p0[t * stride + D + 1], sc, L);
    }
    const int n = min(64, nw - j0);
    const float* pc = p0 + (w + (long long)kCombWaves * j0) * stride;
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sc), j));
#pragma unroll
      for (int x = 0; x < D / 64; ++x)
        acc[x] = fmaf(pc[(long long)j * kCombWaves * stride + x * 64 + lane], s, acc[x]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
#pragma unroll
  for (int x = 0; x < D / 64; ++x) s_red[w][x * 64 + lane] = acc[x];
  if (lane == 0) s_red[w][D] = L;
  __syncthreads();
  if (w != 0) return;
  float Lt = 0.0f;
#pragma unroll
  for (int y = 0; y < kCombWaves; ++y) Lt += s_red[y][D];
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  T* op = (T*)a.o + (long long)bq * D;
#pragma unroll
  for (int x = 0; x < D / 64; ++x) {
    float v = 0.0f;
#pragma unroll
    for (int y = 0; y < kCombWaves; ++y) v += s_red[y][x * 64 + lane];
    op[x * 64 + lane] = (T)(v * inv);
  }
  if (lane == 0) a.lse[bq] = (M + log2f(Lt)) * kLn2;
}

template <typename T, int D, int BLK>
hipError_t launch_attn(const DecArgs& a, int B, hipStream_t st) {
  if (std::is_same<T, __bf16>::value && D == kMD && BLK == kMB && a.G <= 32) {
    hipLaunchKernelGGL(decode_attn_mfma_kernel, dim3((unsigned)(B * a.Hkv), (unsigned)a.T), dim3(64),
                       0, st, a);
  } else {
    const size_t lds = attn_lds<T, D, BLK>(a.G);
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute((const void*)&decode_attn_kernel<T, D, BLK>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_attn_kernel<T, D, BLK>), dim3((unsigned)(B * a.Hkv), (unsigned)a.T),
                       dim3(kAttnThreads), lds, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(B * a.Hq)), dim3(64 * kCombWaves),
                     0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attn_d(const DecArgs& a, int B, int blk, hipStream_t st) {
  if (blk == 16) return launch_attn<T, D, 16>(a, B, st);
  if (blk == 32) return launch_attn<T, D, 32>(a, B, st);
  return launch_attn<T, D, 64>(a, B, st);
}

}  // namespace

// ---------------------------------------------------------------------------
// fixed scratch of the allocation-free decode entry point
// ---------------------------------------------------------------------------
// The tile partials of sas_decode_attn_noalloc live in this array instead of
// a caller workspace.  Each device holds its own copy (from the library's
// code-object load until the process ends).  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked
// up once per device with hipGetSymbolAddress and only that address is
// handed to kernels.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {   // first use on this device (it is current)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t decode_attn_lds_bytes(const DecodeShape& s) {
  const size_t el = s.fp32 ? 4 : 2;
  return 2 * (size_t)s.blk * s.D * el + sizeof(float) * ((size_t)s.G * s.D + (size_t)s.G * s.blk);
}

hipError_t launch_decode_select(const DecodeShape& s, const float* scores, const int32_t* seq_lens,
                                float* tau, int32_t* sel_idx, int32_t* sel_cnt, int32_t* d_status,
                                hipStream_t st) {
  const size_t lds = sizeof(uint32_t) * (size_t)s.cmax;
  if (lds > 60 * 1024) {   // with the kernel's static LDS this passes 64 KB
    const hipError_t e = hipFuncSetAttribute((const void*)&decode_select_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int nthr = s.cmax >= 512 ? kSelMaxThreads : 256;   // 1024 threads: 12.6 -> 10.0 us at 1024 blocks
  hipLaunchKernelGGL(decode_select_kernel, dim3((unsigned)(s.B * s.Hkv)), dim3(nthr), lds,
                     st, scores, seq_lens, tau, sel_idx, sel_cnt, d_status, s.Hkv, s.cmax, s.blk,
                     s.K, s.cap);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const DecodeShape& s, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* sel_idx,
                              const int32_t* sel_cnt, void* o, float* lse, float* part,
                              int32_t* d_status, hipStream_t st) {
  DecArgs a{};
  a.q = q; a.kp = k_pool; a.vp = v_pool; a.bt = block_table; a.seq_lens = seq_lens;
  a.sel_idx = sel_idx; a.sel_cnt = sel_cnt; a.o = o; a.lse = lse; a.part = part;
  a.d_status = d_status;
  a.Hq = s.Hq; a.Hkv = s.Hkv; a.G = s.G; a.cmax = s.cmax; a.pool = s.pool; a.cap = s.cap;
  a.T = s.cap + 1;
  a.c2 = s.scale * kLog2e;
  if (s.fp32) {
    return s.D == 64 ? launch_attn_d<float, 64>(a, s.B, s.blk, st)
                     : launch_attn_d<float, 128>(a, s.B, s.blk, st);
  }
  return s.D == 64 ? launch_attn_d<__bf16, 64>(a, s.B, s.blk, st)
                   : launch_attn_d<__bf16, 128>(a, s.B, s.blk, st);
}

}  // namespace sas
