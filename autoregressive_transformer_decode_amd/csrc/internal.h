// Internal declarations shared by the C-ABI layer (abi.cpp) and the HIP
// kernels (kernels.hip).  Not part of the public interface.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace atd {

constexpr int kMaxTables = 16;
constexpr int kMaxLayers = 64;
constexpr int kGemvMaxRows = 2;      // rows a GEMV launch handles at once
constexpr int kAttnChunkSmall = 128; // keys per attention split, <= 2 rows
constexpr int kAttnChunkLarge = 256; // keys per attention split, > 2 rows
constexpr int kArgmaxChunk = 4096;   // logits per argmax block

// How the rows of a launch map to (slot, position):
//  kRowsStep:    row m -> slot slot0 + m at that slot's current position
//  kRowsPrefill: row m -> slot slot0 at position m
enum RowMode { kRowsStep = 0, kRowsPrefill = 1 };

struct RowMap {
  int mode;
  int slot0;
};

// ---------------------------------------------------------------- GEMV
enum GemvEpilogue { kEpiStore = 0, kEpiResidual = 1, kEpiSwiglu = 2 };

struct GemvArgs {
  const void* W[3];       // row segments [rows_s, K]; segment s ends at seg_end[s]
  const float* bias[3];   // per-segment bias or null (kEpiStore only)
  int seg_end[3];
  const void* W2;         // up-projection [N, K] (kEpiSwiglu)
  const float* x;         // input rows [M, ldx]
  int ldx;
  const float* gain;      // RMSNorm gain [K] when the input is normalised
  float eps;
  float* out;             // output rows [M, ldo]
  int ldo;
  float* y_out;           // normalised input rows [M, K] (block 0 writes), or null
  int K, N, M;
};

// ---------------------------------------------------------------- rows/KV
struct SlotTables {
  void** kv;        // device [max_slots][L][2] cache pointers (K, V)
  int* pos;         // device [max_slots] next write position
  int* cap;         // device [max_slots] capacity (rows)
  int L;
};

struct RopeArgs {
  const float* qkv;   // [M, (Hq + 2 Hkv) D]
  float* q_out;       // [M, Hq, D]
  const float* q_norm;
  const float* k_norm;
  float eps;
  const float* cos_t; // [max_ctx, D/2]
  const float* sin_t;
  SlotTables st;
  RowMap rows;
  int layer, M, Hq, Hkv, D, qk_norm;
};

struct AttnArgs {
  const float* q;     // [M, Hq, D]
  SlotTables st;
  RowMap rows;
  int layer, M, Hq, Hkv, chunk, nsplit_max;
  float scale;
  float* pml;         // [M, Hq, nsplit_max, 2] running max and sum
  float* pacc;        // [M, Hq, nsplit_max, D]
  float* o;           // [M, Hq * D] (combine output)
};

struct EmbedArgs {
  const void* tab[kMaxTables];
  int vocab[kMaxTables];
  int G;
  const int32_t* tok;   // [M, G]
  const float* extra;   // [M, h] or null
  float* out;           // [M, h]
  int h, M;
};

struct ArgmaxArgs {
  const float* z;      // [B, V]
  int B, V;
  uint32_t* seen;      // [B, nwords] or null
  int nwords;
  float penalty;
  int32_t* tok;
  float* margin;
  float* part;         // [B, nblk, 3]
  int nblk;
};

struct KvCopyArgs {
  const void* src[2 * kMaxLayers];
  void* dst[2 * kMaxLayers];
  int n;               // number of buffers (2 L)
  int Hkv, D, rows, s_old, s_new, elem_bytes;
};

// ---------------------------------------------------------------- launchers
// Each returns the first HIP error of its launches (hipSuccess otherwise).
hipError_t launch_embed(const EmbedArgs& a, int bf16, hipStream_t s);
hipError_t launch_gemv(const GemvArgs& a, int epi, bool norm, int bf16, hipStream_t s);
hipError_t launch_rope_append(const RopeArgs& a, int bf16, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int bf16, int D, int r, hipStream_t s);
hipError_t launch_advance(const SlotTables& st, RowMap rows, int M, hipStream_t s);
hipError_t launch_set_slot(const SlotTables& st, int slot, void* const* k, void* const* v,
                           int cap, int pos, int set_ptrs, hipStream_t s);
hipError_t launch_kv_copy(const KvCopyArgs& a, hipStream_t s);
hipError_t launch_argmax(const ArgmaxArgs& a, hipStream_t s);
hipError_t launch_record_token(const int32_t* tok, int32_t* out, int32_t* counter, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);

}  // namespace atd
