// Internal interface between the C-ABI layer (abi.cpp) and the HIP kernels.
// Argument structs are passed to kernels by value; every pointer is a device
// pointer and every stride is in elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/diffattn.h"

namespace da {

struct FwdParams {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  void* out;
  const float* norm_w;  // [dv] or nullptr
  float* lse;           // [2][B][H_s][N] or nullptr
  float* o_maps;        // fp32 [2][B][N][H_s][dv] dense or nullptr: A1 V and A2 V
  const float* lam_dev; // device lambda or nullptr (then lam)
  // packed sequences: sequence s is tokens [cu_seqlens[s], cu_seqlens[s+1]) of
  // batch 0; nullptr = nseq (= B) batches of max_seqlen (= N) tokens each
  const int32_t* cu_seqlens;
  int nseq, max_seqlen;
  int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3], so[3];  // (b, n, head)
  int B, N, Hs, Hn, Hkv, d, dv;
  int g;                // signal heads per noise head
  int causal, normalize;
  float lam, lam_init, eps;
  float sm_scale;       // 1/sqrt(d)
  float sm_scale_log2;  // log2(e)/sqrt(d)
  int16_t nz[DA_MAX_HEADS];      // signal head -> noise head
  int16_t kv[DA_MAX_HEADS];      // signal head -> key/value head
  int16_t members[DA_MAX_HEADS]; // noise group n's signal heads at [n*g, n*g+g)
  // shared-value prefill only: signal heads with the same noise head and the
  // same key/value head form combos of gs heads, combo c at [c*gs, c*gs+gs)
  int gs, ncombo;
  int16_t cmem[DA_MAX_HEADS];
};

struct DecodeParams {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  const int32_t* seq_lens;
  void* out;
  float* ws;            // partials, see decode_bf16.hip
  const float* lam_dev; // device lambda or nullptr (then lam)
  const float* norm_w;
  int64_t sq1[2], sq2[2], so[2];
  int64_t sk1[3], sk2[3], sv[3];
  int B, Lmax, Hs, Hn, Hkv, d, dv;
  int g;                // members per noise group
  int chunk, nchunks;   // keys per partial, partials per (b, group)
  int slots;            // g (map-1 outputs) + u (distinct V heads of a group for map 2)
  int normalize;
  int fp8;              // caches are OCP e4m3 bytes, read as value * scale
  const int32_t* block_table;  // paged caches: [B][max_blocks] or nullptr
  int block_size, max_blocks, num_blocks;
  float k1_scale, k2_scale, v_scale;
  float lam, lam_init, eps, sm_scale_log2;
  int16_t members[DA_MAX_HEADS];   // group n's signal heads at [n*g, n*g+g)
  int16_t kv[DA_MAX_HEADS];        // signal head -> kv head
  int16_t ukv[DA_MAX_HEADS];       // group n's distinct kv heads at [n*g, n*g+u_n)
  int16_t nu[DA_MAX_HEADS];        // u_n per group
  int16_t uidx[DA_MAX_HEADS];      // signal head -> index of its kv head in its group's ukv list
};

// Backward.  Workspace sections (offsets in bytes, each 256-aligned):
//   dop     [B][N][H_s][dv] dense, the gradient at o (head norm undone), in
//           the storage dtype (the MFMA operand of the bf16 passes)
//   rowstat [B][H_s][N] x float4 {lse1 log2(e), lse2 log2(e) - log2|lambda|,
//           D1, sgn D2} with D1 = dop . o1, D2 = dop . o2 per row and
//           -lambda = sgn |lambda| (so 2^(s2 sc - .y) is |lambda| P2)
//   partial [prep workgroups][1 + dv] fp64: per-workgroup sums of -D2 (for
//           dlambda) and of dy c o / r per channel (for dw)
struct BwdParams {
  const void* q1;
  const void* q2;
  const void* k1;
  const void* k2;
  const void* v;
  const float* o_maps;
  const float* lam_dev;  // device lambda or nullptr (then lam)
  const float* lse;
  const void* dout;
  void* gq1;
  void* gq2;
  void* gk1;
  void* gk2;
  void* gv;
  float* dlambda;
  float* dnorm_w;
  const float* norm_w;
  void* dop;
  float* rowstat;
  double* partial;
  int nprep;            // prep workgroups (rows of `partial`)
  int64_t sq1[3], sq2[3], sk1[3], sk2[3], sv[3], sdo[3];
  int64_t sgq1[3], sgq2[3], sgk1[3], sgk2[3], sgv[3];
  int B, N, Hs, Hn, Hkv, d, dv;
  int g, gk;            // signal heads per noise head, per key/value head
  int causal, normalize;
  float lam, lam_init, eps;
  float sm_scale, sm_scale_log2;
  int16_t nz[DA_MAX_HEADS];
  int16_t kv[DA_MAX_HEADS];
  int16_t members[DA_MAX_HEADS];   // noise group n's signal heads at [n*g, n*g+g)
  int16_t kvmembers[DA_MAX_HEADS]; // key/value head k's signal heads at [k*gk, k*gk+gk)
};

// upper bound of BwdParams::nprep: two rounds of three 4-wavefront workgroups
// per compute unit, each wavefront walking many row groups (its next rows'
// loads in flight while it processes the current ones)
constexpr int kBwdPrepBlocks = 1536;

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s);
// per-noise-group prefill for three signal heads per noise head on distinct
// key/value heads (d = 64); gda3_applies says whether a call has that layout
bool gda3_applies(const FwdParams& p);
hipError_t launch_fwd_gda3_bf16(const FwdParams& p, hipStream_t s);
// bf16 prefill for layers whose signal heads share noise and key/value heads
// in combos of 2, 4 or 8 (d = 64, fixed-length batches, nested output
// strides): A2 V formed once per combo (fwd_bf16.hip).  shared_kv_plan fills
// gs, ncombo and cmem and says whether a call has that layout.
bool shared_kv_plan(FwdParams& p);
hipError_t launch_fwd_shared_bf16(const FwdParams& p, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s);
// device address of the current device's fixed decode scratch (DA_DECODE_SCRATCH_BYTES)
hipError_t decode_scratch(float** ptr);
constexpr size_t kDecodeScratchBytes = DA_DECODE_SCRATCH_BYTES;
hipError_t launch_bwd_prep(const BwdParams& p, int dtype, hipStream_t s);
hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t s);
// the score passes for d = 64 with the streamed side in LDS rings (launch_bwd_bf16 uses
// them when bwd_ring_applies)
bool bwd_ring_applies(const BwdParams& p);
hipError_t launch_bwd_ring_bf16(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_finalize(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_zero(const BwdParams& p, hipStream_t s);  // empty input: dlambda = 0, dw = 0
hipError_t launch_lambda_reparam(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int dim,
                                 float lambda_init, float* out, hipStream_t s);
hipError_t launch_lambda_reparam_bwd(const float* lq1, const float* lk1, const float* lq2, const float* lk2, int dim,
                                     const float* dlambda, float* dlq1, float* dlk1, float* dlq2, float* dlk2,
                                     hipStream_t s);

// lambda as the kernels use it: the device value when one is given
__device__ __forceinline__ float lambda_of(const float* dev, float host) { return dev ? *dev : host; }

// workspace floats per (b, group, chunk) for decode
inline int64_t decode_ws_floats_per_chunk(int slots, int dv) { return (int64_t)slots * (dv + 2); }

}  // namespace da
