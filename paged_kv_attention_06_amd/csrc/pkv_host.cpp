// Host side of the C ABI declared in include/pkv.h: argument checks, work
// sizing, launches, the slot-mapping builder and the block allocator.
#include <atomic>
#include <chrono>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <deque>
#include <algorithm>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

// Default shares of the stream decode's waves (see stream_weights).
constexpr int kStreamParityWeight = 0;
constexpr int kStreamAgeWeight = 0;

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PKV_OK;
}

int dtype_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
  }
  return 0;
}

// Checks the descriptor; fills `d` on success.  Sizing queries pass
// need_kv = false and accept a NULL pool pointer.
int check_cache(const pkv_cache* c, pkv::CacheDesc* d, bool need_kv = true) {
  if (!c) return fail(PKV_ERR_NULL, "cache descriptor is NULL");
  if (need_kv && !c->kv) return fail(PKV_ERR_NULL, "cache->kv is NULL");
  if (c->block_size != pkv::kBlockSize)
    return fail(PKV_ERR_DIM, "block_size %d unsupported (must be 16)", c->block_size);
  if (c->num_blocks < 1) return fail(PKV_ERR_DIM, "num_blocks %lld < 1", (long long)c->num_blocks);
  if (c->num_kv_heads < 1) return fail(PKV_ERR_DIM, "num_kv_heads %d < 1", c->num_kv_heads);
  if (c->head_size != 64 && c->head_size != 128)
    return fail(PKV_ERR_DIM, "head_size %d unsupported (64 or 128)", c->head_size);
  const int es = dtype_bytes(c->dtype);
  if (!es) return fail(PKV_ERR_DTYPE, "dtype %d unsupported", c->dtype);
  d->fp8 = c->dtype == PKV_FP8_E4M3;
  d->k_scale = d->v_scale = d->k_inv = d->v_inv = 1.f;
  if (d->fp8) {
    if (!(c->k_scale > 0.f && c->k_scale < INFINITY && c->v_scale > 0.f && c->v_scale < INFINITY))
      return fail(PKV_ERR_RANGE, "fp8 cache scales must be finite and > 0 (k %g, v %g)",
                  (double)c->k_scale, (double)c->v_scale);
    d->k_scale = c->k_scale;
    d->v_scale = c->v_scale;
    d->k_inv = 1.f / c->k_scale;
    d->v_inv = 1.f / c->v_scale;
  }
  d->kv = static_cast<char*>(c->kv);
  d->num_blocks = c->num_blocks;
  d->hkv = c->num_kv_heads;
  d->head_size = c->head_size;
  d->dtype_bytes = es;
  d->block_bytes = (size_t)2 * c->block_size * c->num_kv_heads * c->head_size * es;
  return PKV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// PKV_DEBUG_VALIDATE=1: every entry point copies the device data it is
// about to use (slots, pairs, tables, lengths) to the host after the
// stream's earlier work and checks the preconditions that pkv.h states on
// it (pkv_validate_*), so a bad entry is reported instead of launched.
bool debug_validate() {
  const char* e = std::getenv("PKV_DEBUG_VALIDATE");
  return e && e[0] == '1' && e[1] == '\0';
}

template <typename T>
int fetch(std::vector<T>& dst, const T* src, size_t n, void* stream, const char* what) {
  dst.resize(n > 0 ? n : 1);  // data() of an empty copy is still a valid pointer
  if (n == 0) return PKV_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "PKV_DEBUG_VALIDATE: copy of %s to the host: %s", what,
                hipGetErrorString(e));
  return PKV_OK;
}

// First repeated value of v (indices into the original order), or false.
bool first_repeat(const std::vector<int64_t>& v, int64_t* a, int64_t* b) {
  std::vector<int64_t> idx(v.size());
  for (size_t i = 0; i < v.size(); ++i) idx[i] = (int64_t)i;
  std::sort(idx.begin(), idx.end(), [&v](int64_t x, int64_t y) {
    return v[(size_t)x] != v[(size_t)y] ? v[(size_t)x] < v[(size_t)y] : x < y;
  });
  for (size_t i = 1; i < idx.size(); ++i) {
    if (v[(size_t)idx[i]] == v[(size_t)idx[i - 1]]) {
      *a = idx[i - 1];
      *b = idx[i];
      return true;
    }
  }
  return false;
}

struct Plan {
  int64_t decode_units = 0;
  int64_t full_units = 0;
  int64_t class_count[pkv::kPartClasses] = {0};
  int64_t prefill_tiles = 0;
  int prefill_seqs = 0;
  int64_t max_prefill_q = 0;  // longest q_len of a prefill row
  int64_t prefill_vblocks = 0;
  int64_t num_tokens = 0;
  int64_t stream_steps = 0;  // per kv head: sum over decode rows of steps + setup charge
  int32_t num_seqs = 0;
};

// Validates host lengths and counts the work.  qsl may be NULL (decode).
int plan_attention(const int32_t* qsl, const int32_t* seq_lens, int32_t num_seqs,
                   int32_t max_blocks, int group, Plan* plan) {
  if (!seq_lens) return fail(PKV_ERR_NULL, "host seq_lens is NULL");
  if (num_seqs < 0) return fail(PKV_ERR_DIM, "num_seqs %d < 0", num_seqs);
  if (max_blocks < 0) return fail(PKV_ERR_DIM, "max_blocks_per_seq %d < 0", max_blocks);
  if (qsl && qsl[0] != 0) return fail(PKV_ERR_RANGE, "query_start_loc[0] = %d, must be 0", qsl[0]);
  const int64_t cap = (int64_t)max_blocks * pkv::kBlockSize;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = seq_lens[s];
    const int64_t ql = qsl ? (int64_t)qsl[s + 1] - qsl[s] : 1;
    if (ql < 0) return fail(PKV_ERR_RANGE, "query_start_loc decreases at sequence %d", s);
    if (L < 0 || L > cap)
      return fail(PKV_ERR_RANGE, "seq_lens[%d] = %lld outside [0, %lld]", s, (long long)L,
                  (long long)cap);
    if (qsl && ql > L)
      return fail(PKV_ERR_RANGE, "sequence %d has %lld query rows but length %lld", s,
                  (long long)ql, (long long)L);
    if (ql == 1) {
      if (L > 0) {
        plan->stream_steps += (L + 31) / 32 + pkv::kStreamSetupCost;
        plan->decode_units += (L + pkv::kPartTokens - 1) / pkv::kPartTokens;
        plan->full_units += L / pkv::kPartTokens;
        const int64_t rem = L % pkv::kPartTokens;
        if (rem) plan->class_count[pkv::kPartClasses - (rem + 31) / 32] += 1;
      }
    } else if (ql > 1) {
      const int tq = pkv::prefill_tile_q(group);
      plan->prefill_tiles += (ql + tq - 1) / tq;
      plan->prefill_seqs += 1;
      if (ql > plan->max_prefill_q) plan->max_prefill_q = ql;
      plan->prefill_vblocks += pkv::prefill_vblocks(L);
    }
    plan->num_tokens += ql;
  }
  plan->num_seqs = num_seqs;
  return PKV_OK;
}

// Stream decode sizing: total cost and the most waves a call may use.
int64_t stream_total(const Plan& p, int hkv) { return p.stream_steps * hkv; }
int64_t stream_wave_cap(const Plan& p, int hkv) {
  const int64_t t = stream_total(p, hkv);
  const int64_t w = (t + pkv::kStreamMinCost - 1) / pkv::kStreamMinCost;
  return w < pkv::kMaxStreamWaves ? w : pkv::kMaxStreamWaves;
}

// Shares of the stream decode's waves.  Two effects make waves of equal
// work end at different times (per-wave timestamps on MI355X, 8B GQA batch
// of 256, two waves per SIMD): waves of odd workgroup index (which run on
// the odd XCDs) stream slower, and of the two waves on a SIMD the first
// dispatched (mostly the first half of the grid) runs ahead.  With
// PKV_STREAM_WEIGHTS="x,y" (per mille) the even waves take 1 + x and the odd
// ones 1 - x of an equal share, and the first half of the grid 1 + y, the
// second half 1 - y; 0,0 gives equal shares.  Used only for calls that fill
// every SIMD with two waves (W a multiple of 4).
void stream_weights(int64_t waves, int64_t rounds, bool mixed_call, int* wt, int* half) {
  for (int k = 0; k < 4; ++k) wt[k] = 1024;
  *half = (int)waves;
  int x = kStreamParityWeight, y = kStreamAgeWeight;
  if (const char* e = std::getenv("PKV_STREAM_WEIGHTS")) {
    if (std::sscanf(e, "%d,%d", &x, &y) != 2) x = y = 0;
  }
  if (mixed_call || rounds != 2 || waves % 4 != 0 || x < 0 || y < 0 || x > 200 || y > 200) return;
  if (x == 0 && y == 0) return;
  auto w = [](int sx, int sy, int x, int y) {
    return (int)std::lround(1024.0 * (1000 + sx * x) * (1000 + sy * y) / 1e6);
  };
  wt[0] = w(+1, +1, x, y);
  wt[1] = w(-1, +1, x, y);
  wt[2] = w(+1, -1, x, y);
  wt[3] = 4096 - wt[0] - wt[1] - wt[2];
  *half = (int)(waves / 2);
}

// Epochs of stream-decode counters start at a value that differs between
// runs, so counters left in a reused buffer by another process are stale.
// They are odd (the kernel parks finished counters at 0) and step by 2.
unsigned first_epoch() {
  const auto t = std::chrono::steady_clock::now().time_since_epoch().count();
  return ((unsigned)t ^ (unsigned)((unsigned long long)t >> 32) ^ 0x9E3779B9u) | 1u;
}

// Prefill tiles of calls whose prefill rows are all short (at most 64 query
// rows: speculative verify, small chunks) read bf16 V straight from the pool,
// with P as a bf16 hi + lo pair: such calls are bound by HBM, and the fp16
// copy of V would read V twice and write it once more.  Long chunks keep the
// fp16 copy (one P.V MFMA per step).  PKV_PREFILL_V=bf16|fp16 forces either.
bool prefill_reads_bf16_v(const Plan& p) {
  const char* e = std::getenv("PKV_PREFILL_V");
  if (e && std::strcmp(e, "bf16") == 0) return true;
  if (e && std::strcmp(e, "fp16") == 0) return false;
  return p.max_prefill_q <= 64;
}

// Pure prefill calls whose sequences all have at most 32 / G query rows
// (speculative verify, short chunks) run k_prefill_mq, whose MFMA rows are
// the G heads x 32 / G positions of one sequence.  PKV_PREFILL_MQ=0 sends
// them to the tile kernel instead.
bool prefill_multi_query(const Plan& p, int group) {
  if (p.prefill_tiles == 0 || p.decode_units > 0 || p.max_prefill_q > 32 / group) return false;
  const char* e = std::getenv("PKV_PREFILL_MQ");
  return !(e && std::strcmp(e, "0") == 0);
}

// Pure prefill calls on the fp16-V path whose items (q tile, kv head) each
// get a CU of their own split every item's key tiles between two 4-wave
// groups of one 8-wave workgroup (k_prefill_split); with more items, two
// 4-wave workgroups share a CU (k_prefill_tile).  PKV_PREFILL_SPLIT=1 or 0
// forces either kernel.  Returns 1, 0, or -1 for the automatic choice.
int prefill_split_mode() {
  const char* e = std::getenv("PKV_PREFILL_SPLIT");
  if (e && std::strcmp(e, "1") == 0) return 1;
  if (e && std::strcmp(e, "0") == 0) return 0;
  return -1;
}

// Mixed calls run the prefill tiles on a side stream beside the stream
// decode of their decode rows (one wave per SIMD each), unless
// PKV_MIXED=fused asks for the single k_mixed launch with fixed partitions.
bool mixed_concurrent_enabled() {
  const char* e = std::getenv("PKV_MIXED");
  return !(e && std::strcmp(e, "fused") == 0);
}

// Decode rows use the stream kernel unless PKV_DECODE_SPLIT=units asks for
// fixed 256-token partitions plus a merge launch (in a mixed call: the
// single k_mixed launch, as with PKV_MIXED=fused).
bool stream_decode_enabled() {
  const char* e = std::getenv("PKV_DECODE_SPLIT");
  return !(e && std::strcmp(e, "units") == 0);
}

// Workspace layout: header | decode partials | (256-aligned) fp16 V tiles
// [vblocks][hkv][16 D] | their exponents [hkv][vblocks].  The decode
// partials region is the larger of the two decode paths' needs: fixed
// partitions, acc [units][hq][D] then (m, l) [units][hq][2]; or the stream
// kernel, acc [2 waves][G][D], (m, l) [2 waves][G][2], then (256-aligned)
// counters [num_seqs][hkv] (8 bytes each).
struct WsLayout {
  size_t v_off, exp_off, total;
  size_t st_ml_off, st_ctr_off;  // stream layout (offsets from the start)
};
// stream_waves >= 0 sizes the stream region for that many waves and leaves
// out the fixed partitions' region (the no-allocation entry point, which
// always takes the stream kernel); otherwise both paths fit, for the most
// waves any device may launch.
WsLayout ws_layout(const Plan& p, int hq, int hkv, int D, int64_t stream_waves = -1) {
  WsLayout w{0, 0, 0, 0, 0};
  size_t dec_end = pkv::kWorkspaceHeader;
  if (p.decode_units > 0) {
    const int G = hq / hkv;
    const size_t wc = (size_t)(stream_waves >= 0 ? stream_waves : stream_wave_cap(p, hkv));
    w.st_ml_off = pkv::kWorkspaceHeader + 2 * wc * G * D * sizeof(float);
    w.st_ctr_off = (w.st_ml_off + 2 * wc * G * 2 * sizeof(float) + 255) / 256 * 256;
    const size_t st_total = w.st_ctr_off + (size_t)p.num_seqs * hkv * 8;
    const size_t units = stream_waves >= 0 ? 0
        : pkv::kWorkspaceHeader + (size_t)p.decode_units * hq * (D + 2) * sizeof(float);
    dec_end = st_total > units ? st_total : units;
  }
  if (p.prefill_vblocks == 0) {
    w.total = p.decode_units > 0 ? dec_end : 0;
    return w;
  }
  w.v_off = (dec_end + 255) / 256 * 256;
  w.exp_off = w.v_off + (size_t)p.prefill_vblocks * hkv * pkv::kBlockSize * D * 2;
  w.total = w.exp_off + (size_t)p.prefill_vblocks * hkv * sizeof(int32_t);
  return w;
}


int attention(const pkv_cache* cache, float* out, const void* q, int32_t num_q_heads,
              const int32_t* qsl, const int32_t* seq_lens, const int32_t* h_qsl,
              const int32_t* h_seq_lens, const int32_t* block_tables, int32_t max_blocks,
              int32_t num_seqs, int64_t num_tokens, float scale, void* workspace,
              size_t ws_bytes, void* stream, bool mixed, bool noalloc = false) {
  pkv::CacheDesc c;
  if (int e = check_cache(cache, &c)) return e;
  if (num_q_heads < 1 || num_q_heads % c.hkv != 0)
    return fail(PKV_ERR_DIM, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, c.hkv);
  if (!pkv::supported_group(num_q_heads / c.hkv))
    return fail(PKV_ERR_DIM, "%d query heads per kv head unsupported (1, 2, 4 or 8)",
                num_q_heads / c.hkv);
  if (mixed && !h_qsl) return fail(PKV_ERR_NULL, "host query_start_loc is NULL");
  Plan plan;
  if (int e = plan_attention(mixed ? h_qsl : nullptr, h_seq_lens, num_seqs, max_blocks,
                             num_q_heads / c.hkv, &plan))
    return e;
  if (plan.prefill_tiles > 0 && c.fp8)
    return fail(PKV_ERR_DTYPE, "rows with q_len > 1 need a bf16 cache (this one is fp8)");
  if (plan.prefill_tiles > 0 && !pkv::prefill_supported(num_q_heads / c.hkv, c.dtype_bytes))
    return fail(PKV_ERR_DTYPE,
                "rows with q_len > 1 need a bf16 cache and 1, 2 or 4 query heads per kv head");
  if (mixed && plan.num_tokens != num_tokens)
    return fail(PKV_ERR_RANGE, "query_start_loc[num_seqs] = %lld but num_tokens = %lld",
                (long long)plan.num_tokens, (long long)num_tokens);
  if (plan.num_tokens == 0 && num_seqs == 0) return ok();
  if (!out || !q || !seq_lens || !block_tables || (mixed && !qsl))
    return fail(PKV_ERR_NULL, "a device pointer (out, q, seq_lens, block_tables%s) is NULL",
                mixed ? ", query_start_loc" : "");
  // Stream decode of the decode rows: how many waves.  A decode call whose
  // rows are all empty still runs one wave, which writes their zero rows
  // (and, replayed from a graph after the lengths grew, walks them).
  const bool mixed_call = plan.prefill_tiles > 0 && plan.decode_units > 0;
  const bool decode_rows = plan.decode_units > 0 || (!mixed && num_seqs > 0);
  int64_t waves = 0;
  bool stream_path = false;
  if (decode_rows && (noalloc || stream_decode_enabled() || c.fp8) &&
      (!mixed_call || mixed_concurrent_enabled())) {
    const int G = num_q_heads / c.hkv;
    // Beside prefill tiles the decode keeps one wave per SIMD: a SIMD then
    // holds one prefill wave and one decode wave.
    const int slots = mixed_call ? 4 * pkv::device_cus()
                                 : pkv::decode_stream_slots(c.dtype_bytes, c.head_size, G);
    waves = stream_wave_cap(plan, c.hkv);
    if (waves < 1) waves = 1;
    if (slots > 0 && slots < waves) waves = slots;
    if (const char* e = std::getenv("PKV_STREAM_WAVES")) {  // tuning: cap the waves
      const long long cap = std::atoll(e);
      if (cap > 0 && cap < waves) waves = cap;
    }
    stream_path = slots > 0;
  }
  if (noalloc && !stream_path)
    return fail(PKV_ERR_HIP, "the no-allocation decode needs the device's wave count");
  const WsLayout wl = noalloc ? ws_layout(plan, num_q_heads, c.hkv, c.head_size, waves)
                              : ws_layout(plan, num_q_heads, c.hkv, c.head_size);
  const size_t need = wl.total;
  if (noalloc && need > ws_bytes)
    return fail(PKV_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu "
                "(%d sequences x %d kv heads, %lld waves)",
                need, ws_bytes, num_seqs, c.hkv, (long long)waves);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
  if (debug_validate()) {
    std::vector<int32_t> bt, sl, qv;
    if (int e = fetch(bt, block_tables, (size_t)num_seqs * (size_t)max_blocks, stream,
                      "block_tables"))
      return e;
    if (int e = fetch(sl, seq_lens, (size_t)num_seqs, stream, "seq_lens")) return e;
    if (mixed)
      if (int e = fetch(qv, qsl, (size_t)num_seqs + 1, stream, "query_start_loc")) return e;
    if (int e = pkv_validate_attention(cache, bt.data(), max_blocks, sl.data(), h_seq_lens,
                                       mixed ? qv.data() : nullptr, mixed ? h_qsl : nullptr,
                                       num_seqs))
      return e;
  }
  pkv::AttnDesc a;
  a.out = out;
  a.q = q;
  a.hq = num_q_heads;
  a.block_tables = block_tables;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.h_seq_lens = h_seq_lens;
  a.query_start_loc = mixed ? qsl : nullptr;
  a.num_seqs = num_seqs;
  a.scale = scale * c.k_scale;  // an fp8 cache's K scale folds into the score scale
  a.out_scale = c.v_scale;      // and its V scale into the output
  char* ws = static_cast<char*>(workspace);
  a.ws_acc = ws ? reinterpret_cast<float*>(ws + pkv::kWorkspaceHeader) : nullptr;
  a.ws_ml = a.ws_acc ? a.ws_acc + (size_t)plan.decode_units * num_q_heads * c.head_size : nullptr;
  a.decode_units = plan.decode_units;
  a.full_units = plan.full_units;
  a.class_start[0] = 0;
  for (int k = 0; k < pkv::kPartClasses; ++k) a.class_start[k + 1] = a.class_start[k] + plan.class_count[k];
  a.prefill_tiles = plan.prefill_tiles;
  a.prefill_v_bf16 = prefill_reads_bf16_v(plan);
  a.prefill_mq = prefill_multi_query(plan, num_q_heads / c.hkv);
  a.prefill_split = prefill_split_mode();
  a.prefill_seqs = plan.prefill_seqs;
  a.prefill_vblocks = plan.prefill_vblocks;
  a.ws_v = plan.prefill_vblocks ? ws + wl.v_off : nullptr;
  a.ws_vexp = plan.prefill_vblocks ? reinterpret_cast<int32_t*>(ws + wl.exp_off) : nullptr;
  a.stream_waves = 0;
  a.stream_rounds = 0;
  for (int k = 0; k < 4; ++k) a.stream_wt[k] = 1024;
  a.stream_half = 0;
  if (stream_path) {
    static std::atomic<unsigned> epoch{first_epoch()};
    a.stream_waves = (int)waves;
    a.stream_c0 = pkv::kStreamSetupCost;
    a.stream_epoch = epoch.fetch_add(2, std::memory_order_relaxed);
    // waves per SIMD (rounds of dispatch), which rotate their priority;
    // beside prefill tiles there is one decode wave per SIMD: off
    const int simds = 4 * pkv::device_cus();
    const int64_t rounds = simds > 0 ? (waves + simds - 1) / simds : 0;
    a.stream_rounds = (!mixed_call && rounds > 1) ? (int)(rounds < 4 ? rounds : 4) : 0;
    stream_weights(waves, rounds, mixed_call, a.stream_wt, &a.stream_half);
    // (no decode region when every row is empty: one wave, nothing split)
    const bool region = ws && plan.decode_units > 0;
    a.stream_acc = region ? reinterpret_cast<float*>(ws + pkv::kWorkspaceHeader) : nullptr;
    a.stream_ml = region ? reinterpret_cast<float*>(ws + wl.st_ml_off) : nullptr;
    a.stream_counters =
        region ? reinterpret_cast<unsigned long long*>(ws + wl.st_ctr_off) : nullptr;
  }
  if (c.fp8 && decode_rows && a.stream_waves == 0)
    return fail(PKV_ERR_HIP, "fp8 decode needs the device's wave count (hipGetDevice failed)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.prefill_tiles > 0 && plan.decode_units > 0)
    return hip_status(pkv::launch_mixed_rows(c, a, st), "mixed rows");
  if (plan.prefill_tiles > 0) return hip_status(pkv::launch_prefill_rows(c, a, st), "prefill rows");
  return hip_status(pkv::launch_decode_rows(c, a, st), "decode rows");
}

}  // namespace

// ============================================================================
extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer";
    case PKV_ERR_DIM: return "unsupported or inconsistent dimension";
    case PKV_ERR_DTYPE: return "unsupported dtype";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP error";
    case PKV_ERR_NOMEM: return "no free blocks";
    case PKV_ERR_RANGE: return "index or length out of range";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_version(void) { return 100; }

size_t pkv_block_bytes(const pkv_cache* cache) {
  pkv::CacheDesc c;
  if (check_cache(cache, &c, false)) return 0;
  return c.block_bytes;
}

int pkv_build_slot_mapping(const int32_t* block_tables, int32_t max_blocks,
                           const int32_t* qsl, const int32_t* seq_lens, int32_t num_seqs,
                           int32_t block_size, int64_t* slots) {
  if (block_size != pkv::kBlockSize)
    return fail(PKV_ERR_DIM, "block_size %d unsupported (must be 16)", block_size);
  if (num_seqs < 0 || max_blocks < 0) return fail(PKV_ERR_DIM, "negative count");
  if (num_seqs == 0) return ok();
  if (!block_tables || !qsl || !seq_lens || !slots)
    return fail(PKV_ERR_NULL, "a host pointer is NULL");
  if (qsl[0] != 0) return fail(PKV_ERR_RANGE, "query_start_loc[0] = %d, must be 0", qsl[0]);
  const int64_t cap = (int64_t)max_blocks * block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t q_len = (int64_t)qsl[s + 1] - qsl[s];
    const int64_t L = seq_lens[s];
    if (q_len < 0 || L < q_len || L > cap)
      return fail(PKV_ERR_RANGE, "sequence %d: q_len %lld, length %lld, capacity %lld", s,
                  (long long)q_len, (long long)L, (long long)cap);
    const int32_t* row = block_tables + (int64_t)s * max_blocks;
    for (int64_t i = 0; i < q_len; ++i) {
      const int64_t pos = L - q_len + i;
      const int32_t phys = row[pos / block_size];
      if (phys < 0)
        return fail(PKV_ERR_RANGE, "sequence %d: table entry %lld is negative", s,
                    (long long)(pos / block_size));
      slots[qsl[s] + i] = (int64_t)phys * block_size + pos % block_size;
    }
  }
  return ok();
}

int paged_kv_write(const pkv_cache* cache, const void* k_new, const void* v_new,
                   const int64_t* slot_mapping, int64_t num_tokens, void* stream) {
  pkv::CacheDesc c;
  if (int e = check_cache(cache, &c)) return e;
  if (num_tokens < 0) return fail(PKV_ERR_DIM, "num_tokens %lld < 0", (long long)num_tokens);
  if (num_tokens == 0) return ok();
  if (!k_new || !v_new || !slot_mapping) return fail(PKV_ERR_NULL, "k_new, v_new or slot_mapping is NULL");
  if (debug_validate()) {
    std::vector<int64_t> sv;
    if (int e = fetch(sv, slot_mapping, (size_t)num_tokens, stream, "slot_mapping")) return e;
    if (int e = pkv_validate_slots(cache, sv.data(), num_tokens)) return e;
  }
  return hip_status(pkv::launch_kv_write(c, k_new, v_new, slot_mapping, num_tokens,
                                         static_cast<hipStream_t>(stream)),
                    "paged_kv_write");
}

int block_copy(const pkv_cache* cache, const int64_t* pairs, int64_t num_pairs, void* stream) {
  pkv::CacheDesc c;
  if (int e = check_cache(cache, &c)) return e;
  if (num_pairs < 0) return fail(PKV_ERR_DIM, "num_pairs %lld < 0", (long long)num_pairs);
  if (num_pairs == 0) return ok();
  if (!pairs) return fail(PKV_ERR_NULL, "pairs is NULL");
  if (debug_validate()) {
    std::vector<int64_t> pv;
    if (int e = fetch(pv, pairs, 2 * (size_t)num_pairs, stream, "pairs")) return e;
    if (int e = pkv_validate_block_pairs(pv.data(), num_pairs, c.num_blocks, c.num_blocks, 1))
      return e;
  }
  return hip_status(pkv::launch_block_copy(c, pairs, num_pairs, static_cast<hipStream_t>(stream)),
                    "block_copy");
}

int block_swap(const pkv_cache* cache, void* host_kv, int64_t num_host_blocks,
               const int64_t* pairs, int64_t num_pairs, int32_t direction, void* stream) {
  pkv::CacheDesc c;
  if (int e = check_cache(cache, &c)) return e;
  if (num_pairs < 0 || num_host_blocks < 0)
    return fail(PKV_ERR_DIM, "num_pairs %lld / num_host_blocks %lld < 0", (long long)num_pairs,
                (long long)num_host_blocks);
  if (direction != PKV_SWAP_OUT && direction != PKV_SWAP_IN)
    return fail(PKV_ERR_RANGE, "direction %d is neither PKV_SWAP_OUT nor PKV_SWAP_IN", direction);
  if (num_pairs == 0) return ok();
  if (!host_kv || !pairs) return fail(PKV_ERR_NULL, "host_kv or pairs is NULL");
  if (num_host_blocks < 1) return fail(PKV_ERR_DIM, "the host pool has no blocks");
  if (debug_validate()) {
    std::vector<int64_t> pv;
    if (int e = fetch(pv, pairs, 2 * (size_t)num_pairs, stream, "pairs")) return e;
    const bool out = direction == PKV_SWAP_OUT;
    if (int e = pkv_validate_block_pairs(pv.data(), num_pairs, out ? c.num_blocks : num_host_blocks,
                                         out ? num_host_blocks : c.num_blocks, 0))
      return e;
  }
  void* dev = nullptr;
  if (hipHostGetDevicePointer(&dev, host_kv, 0) != hipSuccess || !dev) {
    (void)hipGetLastError();
    return fail(PKV_ERR_RANGE, "host_kv is not pinned, device-mapped host memory");
  }
  return hip_status(pkv::launch_block_swap(c, static_cast<char*>(dev), pairs, num_pairs,
                                           direction == PKV_SWAP_OUT,
                                           static_cast<hipStream_t>(stream)),
                    "block_swap");
}

int pkv_read_slices(const pkv_cache* cache, const int64_t* slices, int64_t num_slices,
                    int32_t waves, uint32_t* sink, void* stream) {
  pkv::CacheDesc c;
  if (int e = check_cache(cache, &c)) return e;
  if (num_slices < 0 || waves < 1 || waves > (1 << 20))
    return fail(PKV_ERR_DIM, "num_slices %lld, waves %d", (long long)num_slices, waves);
  if (!sink || (num_slices > 0 && !slices)) return fail(PKV_ERR_NULL, "slices or sink is NULL");
  if (debug_validate() && num_slices > 0) {
    std::vector<int64_t> sv;
    if (int e = fetch(sv, slices, (size_t)num_slices, stream, "slices")) return e;
    for (int64_t i = 0; i < num_slices; ++i)
      if (sv[(size_t)i] < 0 || sv[(size_t)i] >= c.num_blocks * c.hkv)
        return fail(PKV_ERR_RANGE, "slices[%lld] = %lld outside [0, num_blocks * num_kv_heads)",
                    (long long)i, (long long)sv[(size_t)i]);
  }
  return hip_status(pkv::launch_read_slices(c, slices, num_slices, waves, sink,
                                            static_cast<hipStream_t>(stream)),
                    "pkv_read_slices");
}

size_t pkv_attention_workspace_bytes(const pkv_cache* cache, int32_t num_q_heads,
                                     const int32_t* h_qsl, const int32_t* h_seq_lens,
                                     int32_t num_seqs) {
  pkv::CacheDesc c;
  if (check_cache(cache, &c, false) || num_q_heads < 1) return 0;
  Plan plan;
  if (num_q_heads % c.hkv != 0 || !pkv::supported_group(num_q_heads / c.hkv)) return 0;
  if (plan_attention(h_qsl, h_seq_lens, num_seqs, INT32_MAX / pkv::kBlockSize,
                     num_q_heads / c.hkv, &plan))
    return 0;
  return ws_layout(plan, num_q_heads, c.hkv, c.head_size).total;
}

int paged_attention_decode(const pkv_cache* cache, float* out, const void* q, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, const int32_t* h_seq_lens, int32_t num_seqs,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return attention(cache, out, q, num_q_heads, nullptr, seq_lens, nullptr, h_seq_lens,
                   block_tables, max_blocks_per_seq, num_seqs, num_seqs, scale, workspace,
                   workspace_bytes, stream, false);
}

int paged_attention_decode_noalloc(const pkv_cache* cache, float* out, const void* q,
                                   int32_t num_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   const int32_t* h_seq_lens, int32_t num_seqs, float scale,
                                   void* stream) {
  char* scratch = nullptr;
  if (hipError_t e = pkv::noalloc_scratch(&scratch))
    return fail(PKV_ERR_HIP, "scratch address (hipGetSymbolAddress): %s", hipGetErrorString(e));
  return attention(cache, out, q, num_q_heads, nullptr, seq_lens, nullptr, h_seq_lens,
                   block_tables, max_blocks_per_seq, num_seqs, num_seqs, scale, scratch,
                   pkv::kNoAllocScratchBytes, stream, false, true);
}

int paged_attention_mixed(const pkv_cache* cache, float* out, const void* q, int32_t num_q_heads,
                          const int32_t* query_start_loc, const int32_t* seq_lens,
                          const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t num_seqs, int64_t num_tokens, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return attention(cache, out, q, num_q_heads, query_start_loc, seq_lens, h_query_start_loc,
                   h_seq_lens, block_tables, max_blocks_per_seq, num_seqs, num_tokens, scale,
                   workspace, workspace_bytes, stream, true);
}

// ---------------------------------------------------------------------------
// preconditions on device data, checked on host copies
// ---------------------------------------------------------------------------
int pkv_layout(void) { return PKV_LAYOUT_HEAD_KV_GRANULE16; }

int pkv_validate_slots(const pkv_cache* cache, const int64_t* slots, int64_t num_tokens) {
  pkv::CacheDesc c;
  if (int e = check_cache(cache, &c, false)) return e;
  if (num_tokens < 0) return fail(PKV_ERR_DIM, "num_tokens %lld < 0", (long long)num_tokens);
  if (num_tokens > 0 && !slots) return fail(PKV_ERR_NULL, "slots is NULL");
  const int64_t cap = c.num_blocks * pkv::kBlockSize;
  std::vector<int64_t> used, tok;
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int64_t sl = slots[t];
    if (sl < 0) continue;
    if (sl >= cap)
      return fail(PKV_ERR_RANGE, "slot_mapping[%lld] = %lld is not below num_blocks * 16 = %lld",
                  (long long)t, (long long)sl, (long long)cap);
    used.push_back(sl);
    tok.push_back(t);
  }
  int64_t a = 0, b = 0;
  if (first_repeat(used, &a, &b))
    return fail(PKV_ERR_RANGE, "slot %lld is written by tokens %lld and %lld",
                (long long)used[(size_t)a], (long long)tok[(size_t)a], (long long)tok[(size_t)b]);
  return ok();
}

int pkv_validate_block_pairs(const int64_t* pairs, int64_t num_pairs, int64_t num_src_blocks,
                             int64_t num_dst_blocks, int32_t same_pool) {
  if (num_pairs < 0 || num_src_blocks < 0 || num_dst_blocks < 0)
    return fail(PKV_ERR_DIM, "negative count");
  if (num_pairs > 0 && !pairs) return fail(PKV_ERR_NULL, "pairs is NULL");
  std::vector<int64_t> dst((size_t)num_pairs);
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int64_t a = pairs[2 * i], b = pairs[2 * i + 1];
    if (a < 0 || a >= num_src_blocks)
      return fail(PKV_ERR_RANGE, "pair %lld: source block %lld outside [0, %lld)", (long long)i,
                  (long long)a, (long long)num_src_blocks);
    if (b < 0 || b >= num_dst_blocks)
      return fail(PKV_ERR_RANGE, "pair %lld: destination block %lld outside [0, %lld)",
                  (long long)i, (long long)b, (long long)num_dst_blocks);
    dst[(size_t)i] = b;
  }
  int64_t x = 0, y = 0;
  if (first_repeat(dst, &x, &y))
    return fail(PKV_ERR_RANGE, "block %lld is the destination of pairs %lld and %lld",
                (long long)dst[(size_t)x], (long long)x, (long long)y);
  if (same_pool) {
    std::vector<int64_t> sorted = dst;
    std::sort(sorted.begin(), sorted.end());
    for (int64_t i = 0; i < num_pairs; ++i) {
      const int64_t a = pairs[2 * i];
      if (std::binary_search(sorted.begin(), sorted.end(), a)) {
        int64_t j = 0;
        while (dst[(size_t)j] != a) ++j;
        return fail(PKV_ERR_RANGE, "block %lld is the destination of pair %lld and the source of "
                    "pair %lld", (long long)a, (long long)j, (long long)i);
      }
    }
  }
  return ok();
}

int pkv_validate_attention(const pkv_cache* cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* h_seq_lens, const int32_t* query_start_loc,
                           const int32_t* h_query_start_loc, int32_t num_seqs) {
  pkv::CacheDesc c;
  if (int e = check_cache(cache, &c, false)) return e;
  if (num_seqs < 0 || max_blocks_per_seq < 0) return fail(PKV_ERR_DIM, "negative count");
  if (num_seqs == 0) return ok();
  if (!block_tables || !seq_lens) return fail(PKV_ERR_NULL, "block_tables or seq_lens is NULL");
  const int32_t* qsl = query_start_loc;
  if (qsl) {
    for (int32_t s = 0; s <= num_seqs; ++s) {
      if (h_query_start_loc && qsl[s] != h_query_start_loc[s])
        return fail(PKV_ERR_RANGE, "query_start_loc[%d] = %d, but %d in the host copy", s,
                    qsl[s], h_query_start_loc[s]);
    }
    if (qsl[0] != 0) return fail(PKV_ERR_RANGE, "query_start_loc[0] = %d, must be 0", qsl[0]);
  }
  const int64_t cap = (int64_t)max_blocks_per_seq * pkv::kBlockSize;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = seq_lens[s];
    if (h_seq_lens && L != h_seq_lens[s])
      return fail(PKV_ERR_RANGE, "seq_lens[%d] = %lld, but %d in the host copy", s, (long long)L,
                  h_seq_lens[s]);
    if (L < 0 || L > cap)
      return fail(PKV_ERR_RANGE, "seq_lens[%d] = %lld outside [0, max_blocks_per_seq * 16 = %lld]",
                  s, (long long)L, (long long)cap);
    if (qsl) {
      const int64_t ql = (int64_t)qsl[s + 1] - qsl[s];
      if (ql < 0 || ql > L)
        return fail(PKV_ERR_RANGE, "sequence %d has %lld query rows and length %lld", s,
                    (long long)ql, (long long)L);
    }
    const int32_t* row = block_tables + (size_t)s * max_blocks_per_seq;
    for (int64_t j = 0; j < (L + pkv::kBlockSize - 1) / pkv::kBlockSize; ++j) {
      if (row[j] < 0 || row[j] >= c.num_blocks)
        return fail(PKV_ERR_RANGE, "block_tables[%d][%lld] = %d outside [0, %lld)", s,
                    (long long)j, row[j], (long long)c.num_blocks);
    }
  }
  return ok();
}

// ---------------------------------------------------------------------------
// host block allocator
// ---------------------------------------------------------------------------
// The free queue is a doubly linked list over block ids, so a block can leave
// it from anywhere in O(1) (a prefix-cache hit on a free block).  Blocks that
// carry a prefix hash keep it (and their place in the cache map) until they
// are taken from the head for a new use.
struct pkv_pool {
  int32_t block_size;
  std::vector<int32_t> ref;
  std::vector<int32_t> prev, next;  // free-queue links (-1 = none)
  std::vector<char> in_free;
  int32_t head = -1, tail = -1;
  int64_t nfree = 0;
  // prefix cache: per block its hash, its parent's hash and its token ids
  std::vector<char> hashed;
  std::vector<uint64_t> hash, parent;
  std::vector<int32_t> toks;  // [num_blocks][block_size], filled on registration
  std::unordered_map<uint64_t, int32_t> by_hash;

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++nfree;
  }
  void push_front(int32_t b) {
    next[b] = head;
    prev[b] = -1;
    if (head >= 0) prev[head] = b; else tail = b;
    head = b;
    in_free[b] = 1;
    ++nfree;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --nfree;
  }
  // Takes the head block for a new use; a cached block loses its hash here.
  int32_t take() {
    const int32_t b = head;
    unlink(b);
    if (!hashed.empty() && hashed[(size_t)b]) {
      auto it = by_hash.find(hash[(size_t)b]);
      if (it != by_hash.end() && it->second == b) by_hash.erase(it);
      hashed[(size_t)b] = 0;
    }
    ref[(size_t)b] = 1;
    return b;
  }
  void drop(int32_t b) {  // one reference less; at zero back to the queue
    if (--ref[(size_t)b] == 0) {
      if (!hashed.empty() && hashed[(size_t)b]) push_back(b); else push_front(b);
    }
  }
  void ensure_cache() {
    if (!hashed.empty()) return;
    const size_t n = ref.size();
    hashed.assign(n, 0);
    hash.assign(n, 0);
    parent.assign(n, 0);
    toks.assign(n * (size_t)block_size, 0);
  }
};

pkv_pool* pkv_pool_create(int64_t num_blocks, const int32_t* free_order, int32_t block_size) {
  if (num_blocks < 1 || num_blocks > INT32_MAX || block_size != pkv::kBlockSize) {
    fail(PKV_ERR_DIM, "pkv_pool_create: num_blocks %lld, block_size %d", (long long)num_blocks,
         block_size);
    return nullptr;
  }
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return nullptr;
  p->block_size = block_size;
  p->ref.assign((size_t)num_blocks, 0);
  p->prev.assign((size_t)num_blocks, -1);
  p->next.assign((size_t)num_blocks, -1);
  p->in_free.assign((size_t)num_blocks, 0);
  std::vector<char> seen;
  if (free_order) seen.assign((size_t)num_blocks, 0);
  for (int64_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : (int32_t)i;
    if (free_order) {
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {
        fail(PKV_ERR_RANGE, "pkv_pool_create: free_order is not a permutation (entry %lld = %d)",
             (long long)i, b);
        delete p;
        return nullptr;
      }
      seen[(size_t)b] = 1;
    }
    p->push_back(b);
  }
  ok();
  return p;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int64_t pkv_pool_num_free(const pkv_pool* pool) { return pool ? pool->nfree : -1; }

int32_t pkv_pool_refcnt(const pkv_pool* pool, int32_t block_id) {
  if (!pool || block_id < 0 || (size_t)block_id >= pool->ref.size()) return -1;
  return pool->ref[(size_t)block_id];
}

int pkv_pool_append(pkv_pool* pool, int32_t* table, int32_t max_blocks, int32_t cur_len,
                    int32_t n_new, int64_t* slots, int64_t* cow_pair) {
  if (!pool || !cow_pair || (!table && max_blocks > 0) || (!slots && n_new > 0))
    return fail(PKV_ERR_NULL, "pkv_pool_append: NULL argument");
  if (cur_len < 0 || n_new < 0 || max_blocks < 0)
    return fail(PKV_ERR_DIM, "pkv_pool_append: negative count");
  const int64_t bs = pool->block_size;
  const int64_t have = (cur_len + bs - 1) / bs;
  const int64_t need = ((int64_t)cur_len + n_new + bs - 1) / bs;
  if (need > max_blocks)
    return fail(PKV_ERR_RANGE, "pkv_pool_append: %lld blocks exceed table capacity %d",
                (long long)need, max_blocks);
  for (int64_t i = 0; i < have; ++i) {
    if (table[i] < 0 || (size_t)table[i] >= pool->ref.size() || pool->ref[(size_t)table[i]] < 1)
      return fail(PKV_ERR_RANGE, "pkv_pool_append: table entry %lld (%d) is not a held block",
                  (long long)i, table[i]);
  }
  const bool into_partial = n_new > 0 && (cur_len % bs) != 0;
  const bool copy = into_partial && pool->ref[(size_t)table[have - 1]] > 1;
  const int64_t fresh = (need - have) + (copy ? 1 : 0);
  if (fresh > pool->nfree)
    return fail(PKV_ERR_NOMEM, "pkv_pool_append: %lld blocks needed, %lld free", (long long)fresh,
                (long long)pool->nfree);
  cow_pair[0] = cow_pair[1] = -1;
  auto take = [pool]() { return pool->take(); };
  if (copy) {
    const int32_t old_b = table[have - 1];
    const int32_t new_b = take();
    pool->ref[(size_t)old_b] -= 1;
    table[have - 1] = new_b;
    cow_pair[0] = old_b;
    cow_pair[1] = new_b;
  }
  for (int64_t i = have; i < need; ++i) table[i] = take();
  for (int64_t i = 0; i < n_new; ++i) {
    const int64_t pos = (int64_t)cur_len + i;
    slots[i] = (int64_t)table[pos / bs] * bs + pos % bs;
  }
  return ok();
}

int pkv_pool_fork(pkv_pool* pool, const int32_t* table, int32_t n, int32_t* out_table) {
  if (!pool || (n > 0 && (!table || !out_table))) return fail(PKV_ERR_NULL, "pkv_pool_fork: NULL argument");
  if (n < 0) return fail(PKV_ERR_DIM, "pkv_pool_fork: negative count");
  for (int32_t i = 0; i < n; ++i) {
    if (table[i] < 0 || (size_t)table[i] >= pool->ref.size() || pool->ref[(size_t)table[i]] < 1)
      return fail(PKV_ERR_RANGE, "pkv_pool_fork: entry %d (%d) is not a held block", i, table[i]);
  }
  for (int32_t i = 0; i < n; ++i) {
    pool->ref[(size_t)table[i]] += 1;
    out_table[i] = table[i];
  }
  return ok();
}

int pkv_pool_release(pkv_pool* pool, const int32_t* table, int32_t n) {
  if (!pool || (n > 0 && !table)) return fail(PKV_ERR_NULL, "pkv_pool_release: NULL argument");
  if (n < 0) return fail(PKV_ERR_DIM, "pkv_pool_release: negative count");
  for (int32_t i = 0; i < n; ++i) {
    if (table[i] < 0 || (size_t)table[i] >= pool->ref.size() || pool->ref[(size_t)table[i]] < 1)
      return fail(PKV_ERR_RANGE, "pkv_pool_release: entry %d (%d) is not a held block", i, table[i]);
  }
  for (int32_t i = n - 1; i >= 0; --i) pool->drop(table[i]);
  return ok();
}

// ---------------------------------------------------------------------------
// prefix caching
// ---------------------------------------------------------------------------
uint64_t pkv_block_hash(uint64_t parent, const int32_t* tokens, int32_t num_tokens) {
  uint64_t h = 0xCBF29CE484222325ull;
  auto mix = [&h](uint64_t v, int nbytes) {
    for (int i = 0; i < nbytes; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= 0x100000001B3ull;
    }
  };
  mix(parent, 8);
  for (int32_t i = 0; i < num_tokens; ++i) mix((uint32_t)tokens[i], 4);
  return h;
}

int pkv_pool_match_prefix(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                          int32_t* table, int32_t max_blocks, int32_t* num_hit) {
  if (!pool || !num_hit || (num_tokens > 0 && !tokens) || (max_blocks > 0 && !table))
    return fail(PKV_ERR_NULL, "pkv_pool_match_prefix: NULL argument");
  if (num_tokens < 0 || max_blocks < 0) return fail(PKV_ERR_DIM, "pkv_pool_match_prefix: negative count");
  *num_hit = 0;
  if (pool->hashed.empty()) return ok();
  const int32_t bs = pool->block_size;
  uint64_t par = 0;
  int32_t n = 0;
  for (int32_t i = 0; i < num_tokens / bs && i < max_blocks; ++i) {
    const int32_t* blk = tokens + (size_t)i * bs;
    const uint64_t h = pkv_block_hash(par, blk, bs);
    auto it = pool->by_hash.find(h);
    if (it == pool->by_hash.end()) break;
    const int32_t b = it->second;
    if (pool->parent[(size_t)b] != par ||
        std::memcmp(&pool->toks[(size_t)b * bs], blk, sizeof(int32_t) * bs) != 0)
      break;
    if (pool->ref[(size_t)b] == 0) pool->unlink(b);
    pool->ref[(size_t)b] += 1;
    table[n++] = b;
    par = h;
  }
  *num_hit = n;
  return ok();
}

int pkv_pool_cache_blocks(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                          const int32_t* table, int32_t num_full_blocks) {
  if (!pool || (num_full_blocks > 0 && (!tokens || !table)))
    return fail(PKV_ERR_NULL, "pkv_pool_cache_blocks: NULL argument");
  if (num_full_blocks < 0 || num_tokens < 0) return fail(PKV_ERR_DIM, "pkv_pool_cache_blocks: negative count");
  const int32_t bs = pool->block_size;
  if ((int64_t)num_full_blocks * bs > num_tokens)
    return fail(PKV_ERR_RANGE, "pkv_pool_cache_blocks: %d full blocks need %lld tokens, %d given",
                num_full_blocks, (long long)num_full_blocks * bs, num_tokens);
  for (int32_t i = 0; i < num_full_blocks; ++i) {
    if (table[i] < 0 || (size_t)table[i] >= pool->ref.size() || pool->ref[(size_t)table[i]] < 1)
      return fail(PKV_ERR_RANGE, "pkv_pool_cache_blocks: entry %d (%d) is not a held block", i,
                  table[i]);
  }
  pool->ensure_cache();
  uint64_t par = 0;
  for (int32_t i = 0; i < num_full_blocks; ++i) {
    const int32_t* blk = tokens + (size_t)i * bs;
    const uint64_t h = pkv_block_hash(par, blk, bs);
    const size_t b = (size_t)table[i];
    if (!pool->hashed[b] && pool->by_hash.find(h) == pool->by_hash.end()) {
      pool->hashed[b] = 1;
      pool->hash[b] = h;
      pool->parent[b] = par;
      std::memcpy(&pool->toks[b * bs], blk, sizeof(int32_t) * bs);
      pool->by_hash.emplace(h, (int32_t)b);
    }
    par = h;
  }
  return ok();
}

}  // extern "C"
