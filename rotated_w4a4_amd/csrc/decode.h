// Internal declarations of the decode-attention launcher (decode.hip).
#pragma once

#include "common.h"

namespace quarot {

struct DecodeTensors {
  const __half* q;
  const int8_t* signs;
  int64_t signs_stride_h;
  const uint8_t* k_q;
  const __half* k_scale;
  const __half* k_zero;  // zero-point mode only
  const uint8_t* v_q;
  const __half* v_scale;
  const __half* v_zero;
  const int32_t* lengths;  // optional
  __half* out;
  float* out_f32;  // optional
  void* workspace;
};

// Position split of a launch: `splits` workgroups of `split_len` positions
// per (batch row, KV head).
void decode_plan(int64_t B, int64_t Hkv, int64_t max_len, int& splits, int& split_len);
int64_t decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_len);
int launch_kv_decode(const DecodeTensors& t, int64_t B, int64_t Hq, int64_t Hkv, int64_t S_cache,
                     int64_t max_len, float sm_scale, int mode, bool cross, hipStream_t stream);

// Device address of this device's copy of the allocation-free entry point's
// scratch array (QUAROT_DECODE_SCRATCH_BYTES), fetched on the first call on
// each device.  Allocates nothing.
int decode_scratch(void** out);

}  // namespace quarot
