/*
 * pkv.h -- paged KV-cache attention for AMD MI355X (gfx950), C ABI.
 *
 * PagedAttention keeps every sequence's keys and values in fixed blocks of
 * 16 tokens that may sit anywhere in a pool; a per-sequence block table maps
 * logical block i to a physical block id, like an OS page table, and the
 * attention kernel walks that table (vLLM 技术内幕 (openeuler), section 2.1;
 * Continuous batching + PagedAttention (juhe.plus), sections 3.2, 3.3, 3.6).
 * New tokens' K/V are scattered to the slots named by a slot_mapping
 * (vLLM 源码精读, section 5.1).
 *
 * Conventions for every entry point
 *  - Pointers documented "device" must point to GPU memory of the current
 *    device; "host" pointers to ordinary CPU memory.  The caller owns every
 *    buffer; the library allocates no device memory and keeps no state
 *    between calls except pkv_pool objects the caller creates and destroys,
 *    and, per device, one side stream and two events that
 *    paged_attention_mixed creates on first use and keeps until the process
 *    ends.
 *  - GPU work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream), asynchronously to the host.  No entry point synchronises or
 *    reads device memory from the host (except in the debug mode below).
 *  - Return value: PKV_OK (0) or a PKV_ERR_* code.  Arguments are checked on
 *    the host before anything is launched; on an error nothing is launched
 *    and pkv_last_error() describes it.  Contents of device buffers (slots,
 *    table entries, lengths) cannot be checked without a copy; they are the
 *    caller's preconditions, stated per call.  With the environment variable
 *    PKV_DEBUG_VALIDATE=1 at the time of a call, the call copies that device
 *    data to the host (after the stream's earlier work: it synchronises the
 *    stream, so it cannot be captured into a graph) and checks it with the
 *    pkv_validate_* functions below; a violation returns PKV_ERR_RANGE and
 *    nothing is launched.
 *
 * KV pool layout (bytes; es = element size, E = 16 / es elements per
 * 16-byte granule, bs = block_size = 16, D = head_size):
 *    pool[num_blocks][num_kv_heads][2][bs * D * es]
 *  index 0 of the "2" is the K tile, 1 the V tile of one (block, kv head):
 *    K tile: element (t, d) at element offset ((d / E) * bs + t) * E + d % E
 *            (16-byte granules of E consecutive d of one token, granule-major)
 *    V tile: element (t, d) at element offset ((t / E) * D + d) * E + t % E
 *            (16-byte granules of E consecutive tokens of one d)
 *  A block therefore holds 2 * bs * num_kv_heads * D * es bytes, the
 *  per-block figure of Inside vLLM ("Engine construction"), and every
 *  (block, kv head) K or V tile is one contiguous run.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,      /* a required pointer is NULL                      */
  PKV_ERR_DIM = 2,       /* unsupported or inconsistent size / count        */
  PKV_ERR_DTYPE = 3,     /* unsupported element type                        */
  PKV_ERR_WORKSPACE = 4, /* workspace smaller than required                 */
  PKV_ERR_HIP = 5,       /* a HIP launch failed (text in pkv_last_error)    */
  PKV_ERR_NOMEM = 6,     /* pkv_pool has too few free blocks                */
  PKV_ERR_RANGE = 7      /* a host-visible index or length is out of range  */
};

/* The pool layout described at the top of this file: pool[block][kv head]
 * [K, V][tile], K tiles granule-major by d, V tiles granule-major by token,
 * 16-byte granules.  pkv_layout() returns it, so a caller that views the pool
 * as a tensor can check that it reads the layout this library writes. */
enum { PKV_LAYOUT_HEAD_KV_GRANULE16 = 1 };
int pkv_layout(void);

/* Element types of a cache.  PKV_FP8_E4M3 stores OCP FP8 E4M3 codes (1 sign
 * bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7F and
 * 0xFF are NaN, largest finite 448) with one scale for K and one for V: a
 * stored code c stands for e4m3(c) * k_scale (or v_scale).  The pages list an
 * FP8 KV cache that halves its memory (vLLM 技术内幕, section 7.2); codes and
 * scales are this library's reading. */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 };

/* Static text for a status code. */
const char* pkv_status_string(int status);
/* Detail of the last error raised on the calling thread ("" if none). */
const char* pkv_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int pkv_version(void);

/* ------------------------------------------------------------ the cache */
typedef struct pkv_cache {
  void* kv;             /* device: the pool, layout above                    */
  int64_t num_blocks;   /* blocks in the pool, >= 1                          */
  int32_t block_size;   /* tokens per block; must be 16                      */
  int32_t num_kv_heads; /* >= 1                                              */
  int32_t head_size;    /* 64 or 128                                         */
  int32_t dtype;        /* PKV_F32, PKV_BF16 or PKV_FP8_E4M3                 */
  float k_scale;        /* PKV_FP8_E4M3: finite, > 0; ignored otherwise      */
  float v_scale;        /* PKV_FP8_E4M3: finite, > 0; ignored otherwise      */
} pkv_cache;

/* Bytes of one block over all kv heads, K and V:
 * 2 * block_size * num_kv_heads * head_size * dtype_bytes
 * (Inside vLLM, "Engine construction").  0 if the descriptor is invalid;
 * cache->kv may be NULL here. */
size_t pkv_block_bytes(const pkv_cache* cache);

/* ------------------------------------------------------ host metadata */
/* Slot of every new token of a step (vLLM 源码精读, section 5.1;
 * juhe.plus section 3.3): sequence s owns rows query_start_loc[s] ..
 * query_start_loc[s+1]-1; row i sits at position
 * p = seq_lens[s] - q_len_s + i and goes to slot
 * block_tables[s][p / block_size] * block_size + p % block_size.
 *   block_tables    host int32 [num_seqs][max_blocks_per_seq], row-major
 *   query_start_loc host int32 [num_seqs + 1], non-decreasing, from 0
 *   seq_lens        host int32 [num_seqs], q_len_s <= seq_lens[s] <=
 *                   max_blocks_per_seq * block_size
 *   slot_mapping    host int64 [query_start_loc[num_seqs]] (output)
 * Errors: PKV_ERR_NULL, PKV_ERR_DIM (block_size != 16, counts < 0),
 * PKV_ERR_RANGE (a length outside the bounds above or a negative table
 * entry on the path). */
int pkv_build_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* query_start_loc, const int32_t* seq_lens,
                           int32_t num_seqs, int32_t block_size, int64_t* slot_mapping);

/* ---------------------------------------------------- KV write (scatter) */
/* Write each new token's K and V rows, all kv heads, into its slot
 * (vLLM 技术内幕 section 2.1: write_to_paged_cache / reshape_and_cache).
 *   k_new, v_new  device [num_tokens][num_kv_heads][head_size], contiguous,
 *                 same element type as the cache (bits are copied as is);
 *                 for a PKV_FP8_E4M3 cache they are bf16 and each value x is
 *                 stored as the E4M3 code nearest to x * (1 / scale) (both
 *                 float32 operations; ties to the even code; magnitudes
 *                 above 448 saturate to 448; NaN stays NaN)
 *   slot_mapping  device int64 [num_tokens]; slot < 0 skips the token.
 * Preconditions on device data: non-negative slots are distinct and
 * < num_blocks * 16.  num_tokens == 0 is a no-op. */
int paged_kv_write(const pkv_cache* cache, const void* k_new, const void* v_new,
                   const int64_t* slot_mapping, int64_t num_tokens, void* stream);

/* ------------------------------------------------------- block copy (COW) */
/* For each pair (src, dst) make block dst a copy of block src, K and V of
 * all kv heads: the copy step of copy-on-write (vLLM 技术内幕 section 2.2;
 * juhe.plus section 3.8).
 *   pairs  device int64 [num_pairs][2] = (src, dst)
 * Preconditions on device data: ids in [0, num_blocks); dsts distinct; no
 * dst is also a src (so every read sees the pre-call contents; a src may
 * repeat).  num_pairs == 0 is a no-op. */
int block_copy(const pkv_cache* cache, const int64_t* pairs, int64_t num_pairs, void* stream);

/* ---------------------------------------------------- block swap (host) */
enum { PKV_SWAP_OUT = 0, PKV_SWAP_IN = 1 };

/* Swap preemption's data move (juhe.plus section 3.9: a preempted
 * sequence's blocks are copied to CPU memory over PCIe and copied back when
 * it resumes; Continuous batching + PagedAttention, swap vs recompute):
 * whole blocks (K and V of all kv heads, pkv_block_bytes each) move between
 * the device pool and a host pool with the same block size.
 *   host_kv    host [num_host_blocks][pkv_block_bytes(cache)], pinned and
 *              device-mapped (hipHostMalloc / torch pin_memory); other memory
 *              is rejected with PKV_ERR_RANGE
 *   pairs      device int64 [num_pairs][2] = (src, dst): a device block id and
 *              a host block id for PKV_SWAP_OUT, the reverse for PKV_SWAP_IN
 *   direction  PKV_SWAP_OUT or PKV_SWAP_IN
 * Preconditions on device data: ids in range; dsts distinct.  The copy is
 * asynchronous on `stream` (host memory is final after the stream syncs).
 * num_pairs == 0 is a no-op. */
int block_swap(const pkv_cache* cache, void* host_kv, int64_t num_host_blocks,
               const int64_t* pairs, int64_t num_pairs, int32_t direction, void* stream);

/* ------------------------------------------------------------ attention */
/* Workspace bytes paged_attention_decode / paged_attention_mixed need for
 * these host lengths: the split-K partials of decode rows (per split row:
 * (head_size + 2) floats per query head and 256-token partition) and, for
 * every sequence with q_len > 1, an fp16 copy of the V tiles of its blocks
 * (rounded up to whole 64-token tiles) with one int32 scale exponent per
 * (block, kv head).  h_query_start_loc may be NULL for a pure decode batch
 * (one query row per sequence); cache->kv may be NULL.  0 on invalid input,
 * and also when no workspace is needed.  A call overwrites the workspace;
 * calls that may overlap need separate workspaces. */
size_t pkv_attention_workspace_bytes(const pkv_cache* cache, int32_t num_q_heads,
                                     const int32_t* h_query_start_loc,
                                     const int32_t* h_seq_lens, int32_t num_seqs);

/* Decode attention: one query row per sequence attends to all seq_lens[s]
 * keys of its sequence through its block table (juhe.plus section 3.6;
 * vLLM 技术内幕 section 2.1).  Query head h reads kv head
 * h / (num_q_heads / num_kv_heads).
 *   out           device float32 [num_seqs][num_q_heads][head_size]
 *   q             device [num_seqs][num_q_heads][head_size], cache dtype
 *                 (bf16 for a PKV_FP8_E4M3 cache, whose K and V are read as
 *                 their codes' values times k_scale and v_scale)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens      device int32 [num_seqs]
 *   h_seq_lens    host copy of seq_lens (sizes the grid; must be equal)
 *   scale         multiplies q.k before the softmax (usually 1/sqrt(D))
 *   workspace     device, >= pkv_attention_workspace_bytes(...) bytes
 * A sequence of length 0 yields a zero row.  Preconditions on device data:
 * the first ceil(seq_lens[s]/16) table entries of row s are valid block
 * ids; the K/V of every position < seq_lens[s] were written.
 * Output is float32 only: the attention outputs are the fp32 accumulations
 * themselves (a bf16 output would round them to 8 significant bits).
 * Graph capture: a captured call replays correctly when the device
 * seq_lens (and block tables) have changed since the capture, as in a
 * decode loop where every length grows by one per step, provided every
 * length stays <= max_blocks_per_seq * 16 and the workspace, which depends
 * only on num_seqs, the head counts and the host lengths' wave count, is
 * the captured one.  The host lengths only size the launch; the kernel
 * plans its work from the device lengths.  (With PKV_DECODE_SPLIT=units the
 * fixed-partition path is used instead, whose plan comes from the host
 * lengths: a captured call of that path is valid only for the lengths it
 * was captured with.) */
int paged_attention_decode(const pkv_cache* cache, float* out, const void* q,
                           int32_t num_q_heads, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* h_seq_lens, int32_t num_seqs, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* paged_attention_decode without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory around the
 * call: code recorded under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and errors as
 * paged_attention_decode (with the same kernels), except:
 *  - the split rows' partials and counters live in a scratch array of
 *    32 MiB that the library's code object holds on each device it runs on
 *    until the process ends; a call whose partials (2 per wave of
 *    num_q_heads / num_kv_heads rows of head_size + 2 floats) and counters
 *    (8 bytes per sequence and kv head) do not fit returns PKV_ERR_WORKSPACE
 *    before launching anything (about 250,000 sequences x kv heads at the
 *    8B shape);
 *  - every call on a device shares that device's array, so calls that may
 *    overlap on one device (several streams, several host threads) race and
 *    must be serialised by the caller;
 *  - PKV_DECODE_SPLIT is ignored (the stream kernel always runs).
 * Nothing in the array needs clearing between calls: split rows count their
 * contributors in counters tagged with each call's own epoch. */
int paged_attention_decode_noalloc(const pkv_cache* cache, float* out, const void* q,
                                   int32_t num_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   const int32_t* h_seq_lens, int32_t num_seqs, float scale,
                                   void* stream);

/* Mixed step: chunked-prefill rows and decode rows in one flattened batch
 * (Inside vLLM, "Forward pass" and "Chunked prefill"; juhe.plus section
 * 4.2).  Sequence s owns query rows query_start_loc[s] ..
 * query_start_loc[s+1]-1; row i sits at position seq_lens[s] - q_len_s + i
 * and sees keys 0..that position (causal).  The step's own K/V must already
 * be written (paged_kv_write on the same stream).
 *   out    device float32 [num_tokens][num_q_heads][head_size]
 *   q      device [num_tokens][num_q_heads][head_size], cache dtype (bf16 for
 *          a PKV_FP8_E4M3 cache; rows with q_len > 1 need a bf16 cache)
 *   query_start_loc, seq_lens: device int32; h_*: equal host copies
 *   num_tokens == query_start_loc[num_seqs]
 * A call with both kinds of rows forks the prefill rows onto the library's
 * side stream of the current device (an event recorded on `stream`) and
 * joins it back (`stream` waits for an event recorded on the side stream),
 * so the work is still ordered by `stream` and can be captured from it.  The
 * side stream and its events are created by the first such call on a device;
 * make that call outside graph capture.  A captured mixed call is valid
 * for the query_start_loc and the prefill rows' lengths it was captured
 * with (they size the prefill grid and the workspace); its decode rows'
 * lengths may change as for paged_attention_decode.
 * Host-checked: q_len_s <= seq_lens[s] <= max_blocks_per_seq * 16. */
int paged_attention_mixed(const pkv_cache* cache, float* out, const void* q,
                          int32_t num_q_heads, const int32_t* query_start_loc,
                          const int32_t* seq_lens, const int32_t* h_query_start_loc,
                          const int32_t* h_seq_lens, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, int32_t num_seqs, int64_t num_tokens,
                          float scale, void* workspace, size_t workspace_bytes, void* stream);

/* ----------------------------------------------------------- measurement */
/* The read rate the decode's access pattern allows on this device: every
 * listed (block, kv head) slice of the pool -- its K and V tiles, 2 * 16 *
 * head_size * dtype_bytes contiguous bytes -- is read once, with the loads
 * the decode uses (1 KiB per instruction, two slices per step per wave with
 * the next step in flight), by `waves` waves that take equal runs of the
 * list; nothing is computed from the values but the XOR of every 32-bit
 * word a wave read, which goes to sink[wave].  Timing this call over the
 * slices a decode batch reads gives that batch's read ceiling.
 *   slices  device int64 [num_slices], each block * num_kv_heads + kv head
 *   sink    device uint32 [waves]
 * Preconditions on device data: slice ids in [0, num_blocks * num_kv_heads)
 * (checked under PKV_DEBUG_VALIDATE=1). */
int pkv_read_slices(const pkv_cache* cache, const int64_t* slices, int64_t num_slices,
                    int32_t waves, uint32_t* sink, void* stream);

/* --------------------------------- preconditions on device data (debug) */
/* Checks of the preconditions the calls above state on device data, run on
 * host copies of that data (PKV_DEBUG_VALIDATE=1 runs them inside the calls;
 * a caller may also run them itself).  PKV_OK, or PKV_ERR_RANGE with the
 * first violation in pkv_last_error(); PKV_ERR_NULL / PKV_ERR_DIM for bad
 * arguments. */

/* paged_kv_write: every slot >= 0 is below num_blocks * 16, and no two
 * tokens share a slot (negative slots are skipped).  slots: host int64
 * [num_tokens]. */
int pkv_validate_slots(const pkv_cache* cache, const int64_t* slots, int64_t num_tokens);

/* block_copy (same_pool = 1) and block_swap (same_pool = 0): sources in
 * [0, num_src_blocks), destinations in [0, num_dst_blocks) and distinct;
 * with same_pool, no block is both a destination and a source.
 * pairs: host int64 [num_pairs][2] = (src, dst). */
int pkv_validate_block_pairs(const int64_t* pairs, int64_t num_pairs, int64_t num_src_blocks,
                             int64_t num_dst_blocks, int32_t same_pool);

/* paged_attention_decode (query_start_loc NULL) and paged_attention_mixed:
 * seq_lens (and query_start_loc) equal their host copies when those are
 * given (NULL skips the comparison); 0 <= seq_lens[s] <= max_blocks_per_seq
 * * 16; q_len_s <= seq_lens[s]; and the first ceil(seq_lens[s] / 16) entries
 * of table row s lie in [0, num_blocks).  Every pointer is host memory:
 * block_tables int32 [num_seqs][max_blocks_per_seq], seq_lens int32
 * [num_seqs], query_start_loc int32 [num_seqs + 1]. */
int pkv_validate_attention(const pkv_cache* cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* h_seq_lens, const int32_t* query_start_loc,
                           const int32_t* h_query_start_loc, int32_t num_seqs);

/* ------------------------------------------------- host block allocator */
/* A pool of block ids with reference counts (vLLM 技术内幕 section 2.1-2.2;
 * Inside vLLM "Scheduler": allocate_slots pops the first n free blocks).
 * Host only; the caller applies the returned copy pairs with block_copy and
 * the returned slots with paged_kv_write. */
typedef struct pkv_pool pkv_pool;

/* free_order (host int32 [num_blocks], a permutation of 0..num_blocks-1,
 * or NULL for ascending) is the order blocks are handed out.  NULL on
 * invalid input or out of host memory. */
pkv_pool* pkv_pool_create(int64_t num_blocks, const int32_t* free_order, int32_t block_size);
void pkv_pool_destroy(pkv_pool* pool);
int64_t pkv_pool_num_free(const pkv_pool* pool);
/* Reference count of a block, -1 if the id is out of range. */
int32_t pkv_pool_refcnt(const pkv_pool* pool, int32_t block_id);

/* Make room for n_new tokens after cur_len cached ones of a sequence whose
 * table (host int32, capacity max_blocks) holds ceil(cur_len/16) ids.
 * If the last block is partly filled and shared (ref > 1) it is first
 * replaced by a fresh block: cow_pair = (old, new), the old block loses one
 * reference (copy-on-write, juhe.plus section 3.8); otherwise cow_pair =
 * (-1, -1).  Then ceil((cur_len+n_new)/16) - ceil(cur_len/16) blocks are
 * appended.  slots (host int64 [n_new]) receives the new tokens' slots.
 * On PKV_ERR_NOMEM / PKV_ERR_RANGE nothing changes. */
int pkv_pool_append(pkv_pool* pool, int32_t* table, int32_t max_blocks, int32_t cur_len,
                    int32_t n_new, int64_t* slots, int64_t* cow_pair);

/* Share a sequence's blocks with a new holder (parallel sampling,
 * juhe.plus section 3.5): every id gains one reference and is copied to
 * out_table (host int32 [num_table_blocks]). */
int pkv_pool_fork(pkv_pool* pool, const int32_t* table, int32_t num_table_blocks,
                  int32_t* out_table);

/* Drop one reference of each listed block, last first; a block whose count
 * reaches 0 goes to the head of the free list (reused first), or to its tail
 * if it carries a prefix-cache hash (see pkv_pool_cache_blocks). */
int pkv_pool_release(pkv_pool* pool, const int32_t* table, int32_t num_table_blocks);

/* ------------------------------------------------------ prefix caching */
/* Prefix caching (Inside vLLM, "Prefix caching"; vLLM 技术内幕 section 4):
 * every full block of a request's token ids gets a chained hash of its
 * parent block's hash and its own token ids; a new request reuses cached
 * blocks from its first block up to the first miss; blocks are registered
 * once their K/V are written.  Released blocks that still carry a hash go to
 * the tail of the free queue (evicted last, the request's first block last
 * of all) and others to its head; a hashed block leaves the cache only when
 * it is taken from the head for a new use (pkv_pool_append). */

/* Hash of one block: 64-bit FNV-1a over `parent` (8 bytes, little-endian;
 * 0 for a request's first block) followed by the num_tokens token ids (4
 * bytes each, little-endian). */
uint64_t pkv_block_hash(uint64_t parent, const int32_t* tokens, int32_t num_tokens);

/* Longest cached prefix of a request's token ids (host int32 [num_tokens];
 * full blocks only, at most max_blocks): its block ids go to table[0 ..
 * *num_hit), each gaining a reference (a free block leaves the free queue).
 * A hit also compares the cached block's parent hash and token ids. */
int pkv_pool_match_prefix(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                          int32_t* table, int32_t max_blocks, int32_t* num_hit);

/* Register the first num_full_blocks blocks of a sequence (host table of
 * held ids) as cached for its token ids.  A block that already carries a
 * hash, or whose hash another block holds, is left as it is. */
int pkv_pool_cache_blocks(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                          const int32_t* table, int32_t num_full_blocks);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
