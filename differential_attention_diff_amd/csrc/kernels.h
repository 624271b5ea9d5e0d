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
  const float* norm_w;
  int64_t sq1[2], sq2[2], so[2];
  int64_t sk1[3], sk2[3], sv[3];
  int B, Lmax, Hs, Hn, Hkv, d, dv;
  int g;                // members per noise group
  int chunk, nchunks;   // keys per partial, partials per (b, group)
  int slots;            // g (map-1 outputs) + u (distinct V heads of a group for map 2)
  int normalize;
  float lam, lam_init, eps, sm_scale_log2;
  int16_t members[DA_MAX_HEADS];   // group n's signal heads at [n*g, n*g+g)
  int16_t kv[DA_MAX_HEADS];        // signal head -> kv head
  int16_t ukv[DA_MAX_HEADS];       // group n's distinct kv heads at [n*g, n*g+u_n)
  int16_t nu[DA_MAX_HEADS];        // u_n per group
  int16_t uidx[DA_MAX_HEADS];      // signal head -> index of its kv head in its group's ukv list
};

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t s);
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t s);

// workspace floats per (b, group, chunk) for decode
inline int64_t decode_ws_floats_per_chunk(int slots, int dv) { return (int64_t)slots * (dv + 2); }

}  // namespace da
