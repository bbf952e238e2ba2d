// Internal declarations shared by the HIP translation units of libsas.
//
// Kernel families:
//   sas_threshold.hip  gate activation + Top-K threshold + selector-score gradient
//   sas_generic.hip    vector-ALU forward / backward for every supported shape
//   sas_mfma_fwd.hip   bf16 matrix-core forward (b = 64, D = 128)
//   sas_mfma_bwd.hip   bf16 matrix-core backward (b = 64, D = 128) and the
//                      selection transpose it needs
//   sas_decode.hip     sparse decode: per-group Top-K select, attention over
//                      the gathered blocks of a paged cache
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sas.h"

namespace sas {

// log2(e) and ln(2): the kernels run the softmax in base 2 (v_exp_f32 is exp2)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Everything a kernel needs to know about one problem (host-validated).
struct Shape {
  int B, Hq, Hkv, G, N, D, blk, C, K, cap;
  int Hs;            // score heads: rows of the gate tables per batch (Hkv or Hq)
  const int32_t* lens;  // device [B] valid tokens per sequence, or nullptr
  const int32_t* cu;    // device [B + 1] token offsets of a packed batch, or nullptr
  long long T;          // packed batch: total tokens
  int fp32;          // 1: tensors are float32, 0: bfloat16
  int o_fp32;        // 1: the forward output o is float32
  float scale;       // sm_scale (already defaulted)
  int act;           // sas_gate_act
  int outer;         // 1: gates scale the value rows after the softmax
  int hard;          // 1: hard Top-K gates with the straight-through estimator
};

// Workspace carve-up of the backward pass (byte offsets, 256-aligned).
struct BwdWorkspace {
  size_t delta;      // float  [B*Hq*N]              Delta: sum of P * dP over a query row
  size_t lsen;       // float  [B*Hq*N]              -LSE log2(e) (-inf: padding row), matrix-core path
  size_t colmask;    // uint32 [B*Hkv*C*W]           column j, bit i*nsh + sl: query block i of
                     //                               score head sl (of the kv head) selected j
  size_t collen;     // int32  [B*Hkv*C]             nsh + #(row, score head) selecting j
  size_t coloff;     // int32  [B*Hkv*C + 1]         prefix of collen
  size_t chunkoff;   // int32  [B*Hkv*C + 1]         prefix of ceil(collen / CH)
  size_t collist;    // int32  [B*Hs*C*(cap+1)]      column lists (codes i*nsh + sl), diagonal first
  size_t partial;    // float  [max_chunks * 2 * 64 * 128]  split dK/dV partial sums
  size_t chunk_rank; // int32  [max_chunks]           rank of a chunk inside its order bucket
  size_t chunk_hist; // int32  [B*Hkv*C + 1]         chunks per (batch, kv head, first row)
  size_t chunk_desc; // int32x4 [max_chunks]          per key-major workgroup: chunk id, column,
                     //                               list offset, entries (bit 30: only chunk)
  size_t total;
  long long max_chunks;
  int words;         // W = ceil(C * nsh / 32), nsh = Hs / Hkv score heads per kv head
};

// Query blocks per pass-B work item of the matrix-core backward (per-head
// gates: G / Gs times as many, at most kColChunkMax, so that a work item
// covers as many 32-row steps as with one gate row per kv group).
constexpr int kColChunk = 16;
constexpr int kColChunkMax = 64;
// query blocks per key-major chunk of problem s
inline int col_chunk(const Shape& s) {
  const int gs = s.Hq / s.Hs;
  const int cc = kColChunk * (s.G / gs);
  return cc < kColChunkMax ? cc : kColChunkMax;
}

bool mfma_path(const Shape& s);
BwdWorkspace bwd_workspace_layout(const Shape& s);

// ---- launchers (return the hipError_t of the last launch) ----
hipError_t launch_threshold(const Shape& s, const float* scores, float* log_gate, float* tau,
                            int32_t* sel_idx, int32_t* sel_cnt, int32_t* d_status,
                            hipStream_t st);
// dscores from the dLogG table.  With sel_idx == nullptr (and always with
// hard gates) the table must be complete (zero outside the written entries).
// Otherwise the table holds valid values only at each row's selected blocks,
// and this call also writes the rest of it as 0.
hipError_t launch_dscores(const Shape& s, float* dlog_gate, const float* log_gate,
                          float* dscores, const int32_t* sel_idx, const int32_t* sel_cnt,
                          hipStream_t st);

hipError_t launch_fwd_generic(const Shape& s, const void* q, const void* k, const void* v,
                              const float* log_gate, const int32_t* sel_idx,
                              const int32_t* sel_cnt, void* o, float* lse, hipStream_t st);
// Backward stages.  Stage "dq": dq, Delta (sum of P dP per query row, in the
// workspace) and, on the matrix-core path, the selection transpose.  Stage
// "dkdv": dk, dv, dlog_gate (+ dscores if non-null).
struct BwdPtrs {
  const void* q; const void* k; const void* v; const void* o; const void* d_o;
  const float* lse; const float* log_gate; const int32_t* sel_idx; const int32_t* sel_cnt;
  void* dq; void* dk; void* dv; float* dlog_gate; float* dscores;
};
hipError_t launch_bwd_dq_generic(const Shape& s, const BwdPtrs& p, char* ws,
                                 const BwdWorkspace& wl, hipStream_t st);
hipError_t launch_bwd_dkdv_generic(const Shape& s, const BwdPtrs& p, char* ws,
                                   const BwdWorkspace& wl, hipStream_t st);
hipError_t launch_ste_dropped(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl,
                              hipStream_t st);
hipError_t launch_bwd_dq_mfma(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl,
                              hipStream_t st);
hipError_t launch_bwd_dkdv_mfma(const Shape& s, const BwdPtrs& p, char* ws,
                                const BwdWorkspace& wl, hipStream_t st);

// ---- sparse decode (sas_decode.hip) ----
struct DecodeShape {
  int B, Hq, Hkv, G, D, blk, cmax, pool, K, cap;
  int fp32;
  float scale;
};
size_t decode_attn_lds_bytes(const DecodeShape& s);
// Fixed device scratch of the allocation-free decode entry point: bytes, and
// its device address on the current device (looked up on first use).
constexpr size_t kDecodeScratchBytes = SAS_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch(void** ptr);
hipError_t launch_decode_select(const DecodeShape& s, const float* scores, const int32_t* seq_lens,
                                float* tau, int32_t* sel_idx, int32_t* sel_cnt, int32_t* d_status,
                                hipStream_t st);
// part: workspace of B * Hkv * (cap + 1) * G * (D + 2) floats (tile partials)
hipError_t launch_decode_attn(const DecodeShape& s, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* sel_idx,
                              const int32_t* sel_cnt, void* o, float* lse, float* part,
                              int32_t* d_status, hipStream_t st);

hipError_t launch_fwd_mfma(const Shape& s, const void* q, const void* k, const void* v,
                           const float* log_gate, const int32_t* sel_idx, const int32_t* sel_cnt,
                           void* o, float* lse, hipStream_t st);

// ---- device helpers ----
// Hardware workgroup ids are dealt round-robin over the 8 XCDs (each with its
// own L2).  Map them so that each XCD receives a contiguous range of logical
// work units (consecutive query blocks of one kv head share K/V blocks).
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int q = nwg >> 3, r = nwg & 7;
  const int x = bid & 7, idx = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + idx;
}

// The hardware workgroup id that xcd_remap maps to logical id u (its inverse).
__device__ __forceinline__ int xcd_unmap(int u, int nwg) {
  const int q = nwg >> 3, r = nwg & 7;
  const int x = u < r * (q + 1) ? u / (q + 1) : r + (u - r * (q + 1)) / q;
  const int start = x * q + min(x, r);
  return (u - start) * 8 + x;
}

// Swizzle of the 16-byte chunks of a row-major LDS tile with 256-byte rows:
// chunk c of row r is stored in slot c ^ slot16(r).  gfx950's LDS has 64
// banks; a 16-byte read is served 16 lanes (256 bytes) at a time and an
// 8-byte or transposed read 16 lanes (128 bytes) at a time.  slot16 permutes
// the low four bits of r, so (a) sixteen consecutive rows read at one chunk
// hit sixteen different slots, and (b) the four rows of an aligned group,
// read as 32-byte chunk pairs by a transposed read, hit four different pairs.
__device__ __forceinline__ int slot16(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const char* lptr;
  return (unsigned)(uintptr_t)(lptr)p;
}

// Batches of transposed LDS reads (ds_read_b64_tr_b16) issued back to back
// and awaited inside the same asm block.  Written as asm because the
// compiler, unable to tell these reads apart from the addresses that pending
// global -> LDS copies write, would otherwise wait for every copy in flight
// (including the next tile's prefetch) before the first of them.
typedef uint32_t tr_u32x2 __attribute__((ext_vector_type(2)));

// r[4k + x] = read at a_k + x * 4096 bytes (k = 0, 1; x = 0..3)
__device__ __forceinline__ void tr_read_2x4(unsigned a0, unsigned a1, tr_u32x2 (&r)[8]) {
  __asm__ volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:8192\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:12288\n\t"
      "ds_read_b64_tr_b16 %4, %9\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %9 offset:8192\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:12288\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a0), "v"(a1)
      : "memory");
}

// r[2k + x] = read at a_k + x * 4096 bytes (k = 0..3; x = 0, 1)
__device__ __forceinline__ void tr_read_4x2(unsigned a0, unsigned a1, unsigned a2, unsigned a3,
                                            tr_u32x2 (&r)[8]) {
  __asm__ volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:4096\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

// Asynchronous global -> LDS copies (global_load_lds_dword[x4]): every lane
// copies 4 / 16 bytes from its own global address to lds_base + 4 / 16 * lane
// (lds_base wave-uniform, in M0).  Issued from asm so that the compiler does
// not track them: it would otherwise make every later LDS access wait for all
// copies in flight, prefetches included.  Completion is the caller's: an
// explicit s_waitcnt vmcnt before the barrier that publishes the data (any
// vmcnt wait the compiler places for its own loads only waits longer).
__device__ __forceinline__ void dma16(const void* g, unsigned lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_base);
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(g), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, unsigned lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_base);
  __asm__ volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                   :: "v"(g), "s"(m0) : "memory", "m0");
}

// Same copies with a wave-uniform 64-bit base (SGPRs) and a per-lane 32-bit
// byte offset: the address arithmetic stays in scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16s(const void* base, unsigned voff, unsigned lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_base);
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(voff), "s"(uniform_ptr(base)), "s"(m0) : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* base, unsigned voff, unsigned lds_base) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_base);
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                   :: "v"(voff), "s"(uniform_ptr(base)), "s"(m0) : "memory", "m0");
}

// Forces the loads that produced x to complete here (an asm use of x).
template <typename T>
__device__ __forceinline__ void settle(const T& x) { __asm__ volatile("" ::"v"(x)); }

__device__ __forceinline__ int lane_value(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

}  // namespace sas
