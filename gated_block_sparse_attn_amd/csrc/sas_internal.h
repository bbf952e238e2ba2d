// Internal declarations shared by the HIP translation units of libsas.
//
// Kernel families:
//   sas_threshold.hip  gate activation + Top-K threshold + selector-score gradient
//   sas_generic.hip    vector-ALU forward / backward for every supported shape
//   sas_mfma_fwd.hip   bf16 matrix-core forward (b = 64, D = 128)
//   sas_mfma_bwd.hip   bf16 matrix-core backward (b = 64, D = 128) and the
//                      selection transpose it needs
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sas {

// log2(e) and ln(2): the kernels run the softmax in base 2 (v_exp_f32 is exp2)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Everything a kernel needs to know about one problem (host-validated).
struct Shape {
  int B, Hq, Hkv, G, N, D, blk, C, K, cap;
  int fp32;          // 1: tensors are float32, 0: bfloat16
  int o_fp32;        // 1: the forward output o is float32
  float scale;       // sm_scale (already defaulted)
};

// Workspace carve-up of the backward pass (byte offsets, 256-aligned).
struct BwdWorkspace {
  size_t delta;      // float  [B*Hq*N]              rowsum(O * dO)
  size_t dlg_part;   // float  [parts*B*Hkv*C*(cap+1)] per-head-chunk dLogG partials
  size_t colmask;    // uint32 [B*Hkv*C*W]           bit (j, i): row i selected block j
  size_t collen;     // int32  [B*Hkv*C]             1 + #rows selecting column j
  size_t coloff;     // int32  [B*Hkv*C + 1]         prefix of collen
  size_t chunkoff;   // int32  [B*Hkv*C + 1]         prefix of ceil(collen / CH)
  size_t collist;    // int32  [B*Hkv*C*(cap+1)]     column lists, diagonal first
  size_t partial;    // float  [max_chunks * 2 * 64 * 128]  split dK/dV partial sums
  size_t chunk_rank; // int32  [max_chunks]           rank of a chunk inside its order bucket
  size_t chunk_hist; // int32  [B*Hkv*C + 1]         chunks per (batch, kv head, first row)
  size_t chunk_order;// int32  [max_chunks]           chunk ids sorted by that key
  size_t total;
  long long max_chunks;
  int words;         // W = ceil(C / 32)
};

// Query blocks per pass-B work item of the matrix-core backward.
constexpr int kColChunk = 16;

bool mfma_path(const Shape& s);
int bwd_head_parts(int G);   // head chunks (of 4, 2, 1) the matrix-core passes use
BwdWorkspace bwd_workspace_layout(const Shape& s);

// ---- launchers (return the hipError_t of the last launch) ----
hipError_t launch_threshold(const Shape& s, const float* scores, float* log_gate, float* tau,
                            int32_t* sel_idx, int32_t* sel_cnt, int32_t* d_status,
                            hipStream_t st);
hipError_t launch_dscores(const Shape& s, const float* dlog_gate, const float* log_gate,
                          float* dscores, hipStream_t st);

hipError_t launch_fwd_generic(const Shape& s, const void* q, const void* k, const void* v,
                              const float* log_gate, const int32_t* sel_idx,
                              const int32_t* sel_cnt, void* o, float* lse, hipStream_t st);
// Backward stages.  Stage "dq": Delta, dq, dlog_gate (+ dscores if non-null)
// and, on the matrix-core path, the selection transpose.  Stage "dkdv": dk, dv.
struct BwdPtrs {
  const void* q; const void* k; const void* v; const void* o; const void* d_o;
  const float* lse; const float* log_gate; const int32_t* sel_idx; const int32_t* sel_cnt;
  void* dq; void* dk; void* dv; float* dlog_gate; float* dscores;
};
hipError_t launch_bwd_dq_generic(const Shape& s, const BwdPtrs& p, char* ws,
                                 const BwdWorkspace& wl, hipStream_t st);
hipError_t launch_bwd_dkdv_generic(const Shape& s, const BwdPtrs& p, char* ws,
                                   const BwdWorkspace& wl, hipStream_t st);
hipError_t launch_bwd_dq_mfma(const Shape& s, const BwdPtrs& p, char* ws, const BwdWorkspace& wl,
                              hipStream_t st);
hipError_t launch_bwd_dkdv_mfma(const Shape& s, const BwdPtrs& p, char* ws,
                                const BwdWorkspace& wl, hipStream_t st);

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

}  // namespace sas
