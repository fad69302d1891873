// Internal interface between the C-ABI host layer (pkv_host.cpp) and the
// HIP kernels (pkv_kernels.hip).  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockSize = 16;
// Split-K partition length of the decode kernel, in tokens (a multiple of
// the 64 tokens one wave covers per step).  The workspace size depends on it.
constexpr int kPartTokens = 256;
// Query positions per prefill workgroup: its 4 waves of 32 query rows cover
// the G query heads of one kv head, so 128 / G positions.
constexpr int prefill_tile_q(int g) { return 128 / g; }
// Size classes of the short last partitions (by 32-token steps).
constexpr int kPartClasses = kPartTokens / 32;
// Stream decode: setup charge of an item in 32-token steps, the least cost
// one wave's range is given, and the most waves one call may use (the
// workspace holds two partials per wave).
constexpr int kStreamSetupCost = 1;
constexpr int kStreamMinCost = 8;
constexpr int kMaxStreamWaves = 4096;
// Bytes at the start of the attention workspace before the partials.
constexpr size_t kWorkspaceHeader = 256;
// Blocks of a prefill sequence of length L whose V the prefill path converts
// to fp16 (whole 64-key tiles).
inline int64_t prefill_vblocks(int64_t L) { return 4 * ((L + 4 * kBlockSize - 1) / (4 * kBlockSize)); }

struct CacheDesc {
  char* kv;
  int64_t num_blocks;
  int hkv;
  int head_size;
  int dtype_bytes;
  size_t block_bytes;  // 2 * 16 * hkv * D * es
  bool fp8;            // E4M3 codes; new rows and queries are bf16
  float k_scale, v_scale;  // fp8: a code stands for e4m3 value * scale
  float k_inv, v_inv;      // fp8: 1 / scale in float32, the write's multiplier
};

struct AttnDesc {
  float* out;
  const void* q;
  int hq;
  const int32_t* block_tables;
  int max_blocks;
  const int32_t* seq_lens;
  const int32_t* h_seq_lens;       // host copy (valid during the call)
  const int32_t* query_start_loc;  // nullptr: pure decode, row s = sequence s
  int num_seqs;
  float scale;
  float out_scale;                 // multiplies the output (the V scale of an fp8 cache)
  float* ws_acc;                   // [units][hq][D]
  float* ws_ml;                    // [units][hq][2]
  int64_t decode_units;            // split-K work units over all decode rows
  int64_t full_units;              // of which full kPartTokens partitions
  int64_t class_start[kPartClasses + 1];  // partial units before size class k
  int64_t prefill_tiles;           // prefill q-tiles over all prefill rows
  bool prefill_v_bf16;             // prefill tiles read bf16 V from the pool (no fp16 copy)
  bool prefill_mq;                 // pure prefill, every q_len <= 32 / G: k_prefill_mq
  int prefill_split;               // pure prefill, fp16 V: k_prefill_split 1 always, 0 never,
                                   // -1 when every item has a CU of its own
  int prefill_seqs;                // sequences with more than one query row
  int64_t prefill_vblocks;         // blocks of the prefill sequences, each rounded up to 4
  char* ws_v;                      // fp16 V tiles of those blocks [vblock][hkv][16 * D]
  int32_t* ws_vexp;                // their power-of-two scale exponents [hkv][vblock]
  // stream decode (stream_waves > 0 selects it)
  int stream_waves;                // ranges / waves of the launch
  int stream_c0;                   // setup charge per item
  unsigned stream_epoch;           // distinct per call
  int stream_rounds;               // > 1: waves per SIMD, which rotate their issue priority
  int stream_wt[4];                // shares of the waves (see StreamParams)
  int stream_half;
  unsigned long long* stream_counters;  // [num_seqs][hkv]
  float* stream_acc;               // [2 * waves][G][D]
  float* stream_ml;                // [2 * waves][G][2]
};

hipError_t launch_kv_write(const CacheDesc& c, const void* k_new, const void* v_new,
                           const int64_t* slots, int64_t num_tokens, hipStream_t stream);
hipError_t launch_block_copy(const CacheDesc& c, const int64_t* pairs, int64_t num_pairs,
                             hipStream_t stream);
// Whole blocks between the device pool and a device-mapped host pool.
hipError_t launch_block_swap(const CacheDesc& c, char* host_dev_ptr, const int64_t* pairs,
                             int64_t num_pairs, bool to_host, hipStream_t stream);
// Read probe: every listed (block, kv head) slice once, XOR per wave.
hipError_t launch_read_slices(const CacheDesc& c, const int64_t* slices, int64_t n, int waves,
                              uint32_t* sink, hipStream_t stream);
// Decode rows (one query row per sequence, or the q_len == 1 rows of a mixed
// batch): split-K partition pass, then the merge of multi-partition rows.
hipError_t launch_decode_rows(const CacheDesc& c, const AttnDesc& a, hipStream_t stream);
// Prefill rows of a mixed batch (q_len > 1) when it has no decode rows: MFMA tiles.
hipError_t launch_prefill_rows(const CacheDesc& c, const AttnDesc& a, hipStream_t stream);
// A batch with both kinds of rows.  With stream_waves > 0: the prefill
// tiles on the library's side stream (one workgroup per CU) beside the
// stream decode of the decode rows on `stream`, joined back into `stream`.
// Otherwise one launch in which prefill tiles and fixed decode partitions
// share the GPU, then the merge of split decode rows.
hipError_t launch_mixed_rows(const CacheDesc& c, const AttnDesc& a, hipStream_t stream);

// Bytes of the scratch array of paged_attention_decode_noalloc (one per
// device), and its device address on the current device (looked up once per
// device; the array's name is not usable as an address in host code).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(char** ptr);

bool supported_group(int g);
// Waves of the stream decode kernel the current device holds at once (0 if
// it cannot be queried).
int decode_stream_slots(int dtype_bytes, int D, int G);
// Compute units of the current device (0 if they cannot be queried).
int device_cus();
// Group sizes the mixed path's prefill rows support (bf16 caches only).
inline bool prefill_supported(int g, int dtype_bytes) {
  return dtype_bytes == 2 && (g == 1 || g == 2 || g == 4);
}

}  // namespace pkv
