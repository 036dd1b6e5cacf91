// Serving-policy simulator: periodic window compression against
// threshold-triggered whole-cache compression, under a KV memory cap and a
// concurrency limit ("Technical Summary: Kara", Problem Statement 1 and
// Methodology 3; paper, Fig. 1 caption: compression frees memory so more
// sequences decode at once, and threshold triggering lowers throughput as
// concurrency grows).  Host only; the per-step costs are inputs, taken from
// measured kernel timings.
//
// One call simulates one policy over a seeded request trace, step by step:
//   1. admission: waiting requests enter in order while fewer than max_batch
//      run and the pool has the prompt's blocks plus one spare block;
//   2. decode: every running sequence, in admission order, appends one token
//      (taking a new block when its length is a multiple of the block size;
//      with no free block it stalls for the step); if every running sequence
//      stalled, the most recently admitted one is preempted: its blocks are
//      freed and it goes back to the front of the queue, to restart from its
//      prompt (its generated tokens are wasted);
//   3. finished sequences (all their tokens generated) leave and free blocks;
//   4. compression (none for the uncompressed baseline):
//        periodic   at steps that are multiples of the period, every running
//                   sequence whose trailing window lies after its watermark
//                   (length - watermark >= W) keeps R of the window's first
//                   W - B tokens: length L -> L - (W - B) + R, the tail from
//                   the window's first block is rewritten into
//                   ceil((p + R + B) / bs) blocks (p = (L - W) mod bs), and the
//                   watermark moves to the new length - B;
//        threshold  every running sequence whose length reached the threshold
//                   keeps `keep` tokens of its whole cache (ceil(keep / bs)
//                   blocks);
//   5. step time = decode_ms_fixed + decode_ms_per_token * (cached tokens of
//      the running sequences before the step) + the step's compression cost
//      (periodic: compress_ms_per_seq per sequence; threshold:
//      compress_ms_per_key per cached key scored, i.e. times its length).
// Generation lengths come from SplitMix64 (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", 2014) on seed + request index.

#include "kara.h"

#include <algorithm>
#include <cstdint>
#include <deque>
#include <vector>

namespace {

uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Seq {
  int32_t request;
  int64_t len, gen_left, generated, watermark, blocks;
};

}  // namespace

extern "C" {

int32_t kara_sim_gen_length(const kara_sim_config* c, int32_t request) {
  const uint64_t span = (uint64_t)(c->gen_max - c->gen_min + 1);
  return c->gen_min + (int32_t)(splitmix64(c->seed + (uint64_t)request) % span);
}

kara_status kara_policy_sim(const kara_sim_config* c, kara_sim_result* r, int32_t* active_per_step,
                            int32_t* compressions_per_step, double* ms_per_step) {
  if (!c || !r) return KARA_E_INVAL;
  const bool periodic = c->policy == KARA_POLICY_PERIODIC;
  const bool threshold = c->policy == KARA_POLICY_THRESHOLD;
  if ((!periodic && !threshold && c->policy != KARA_POLICY_NONE) || c->n_requests < 0 ||
      c->max_batch < 1 || c->cap_blocks < 1 || c->block_size < 1 || c->prompt_len < 1 || c->gen_min < 1 ||
      c->gen_max < c->gen_min || c->max_steps < 0)
    return KARA_E_INVAL;
  if (periodic && (c->window < 1 || c->protect < 0 || c->protect >= c->window || c->budget < 1 ||
                   c->budget > c->window - c->protect || c->period < 1))
    return KARA_E_INVAL;
  if (threshold && (c->keep < 1 || c->threshold <= c->keep)) return KARA_E_INVAL;
  const int64_t bs = c->block_size;
  if (cdiv(c->prompt_len, bs) + 1 > c->cap_blocks) return KARA_E_INVAL;   // no request could ever start

  *r = kara_sim_result{};
  std::vector<Seq> run;
  std::deque<int32_t> waiting;
  for (int32_t i = 0; i < c->n_requests; ++i) waiting.push_back(i);
  int64_t free_blocks = c->cap_blocks;
  double active_sum = 0.0;
  int64_t step = 0;
  while (step < c->max_steps && (!waiting.empty() || !run.empty())) {
    ++step;
    // 1. admission
    while (!waiting.empty() && (int32_t)run.size() < c->max_batch) {
      const int64_t need = cdiv(c->prompt_len, bs);
      if (free_blocks < need + 1) break;
      free_blocks -= need;
      const int32_t q = waiting.front();
      waiting.pop_front();
      run.push_back(Seq{q, c->prompt_len, kara_sim_gen_length(c, q), 0, 0, need});
    }
    // 2. decode (cost from the cache before the step)
    int64_t cached = 0;
    for (const Seq& s : run) cached += s.len;
    double ms = c->decode_ms_fixed + c->decode_ms_per_token * (double)cached;
    int64_t advanced = 0;
    for (Seq& s : run) {
      if (s.len % bs == 0) {
        if (free_blocks < 1) {
          ++r->stalls;
          continue;
        }
        --free_blocks;
        ++s.blocks;
      }
      ++s.len;
      --s.gen_left;
      ++s.generated;
      ++r->tokens;
      ++advanced;
    }
    if (!run.empty() && advanced == 0) {
      const Seq& v = run.back();
      free_blocks += v.blocks;
      r->wasted += v.generated;
      ++r->preemptions;
      waiting.push_front(v.request);
      run.pop_back();
    }
    // 3. finished sequences leave
    std::vector<Seq> keep_run;
    keep_run.reserve(run.size());
    for (const Seq& s : run) {
      if (s.gen_left <= 0) free_blocks += s.blocks;
      else keep_run.push_back(s);
    }
    run.swap(keep_run);
    // 4. compression
    int32_t n_comp = 0;
    const double ms_before = ms;
    if (periodic) {
      if (step % c->period == 0) {
        const int64_t W = c->window, B = c->protect, R = c->budget;
        for (Seq& s : run) {
          if (s.len - s.watermark < W) continue;
          const int64_t f0 = (s.len - W) / bs, p = (s.len - W) % bs;
          const int64_t after = f0 + cdiv(p + R + B, bs);
          free_blocks += s.blocks - after;
          s.blocks = after;
          s.len = s.len - (W - B) + R;
          s.watermark = s.len - B;
          ms += c->compress_ms_per_seq;
          ++n_comp;
        }
      }
    } else if (threshold) {
      for (Seq& s : run) {
        if (s.len < c->threshold) continue;
        ms += c->compress_ms_per_key * (double)s.len;
        const int64_t after = cdiv(c->keep, bs);
        free_blocks += s.blocks - after;
        s.blocks = after;
        s.len = c->keep;
        ++n_comp;
      }
    }
    r->compressions += n_comp;
    r->compress_ms += ms - ms_before;
    const int64_t used = c->cap_blocks - free_blocks;
    r->peak_blocks = std::max(r->peak_blocks, used);
    active_sum += (double)run.size();
    r->total_ms += ms;
    if (active_per_step) active_per_step[step - 1] = (int32_t)run.size();
    if (compressions_per_step) compressions_per_step[step - 1] = n_comp;
    if (ms_per_step) ms_per_step[step - 1] = ms;
  }
  r->steps = step;
  r->finished = c->n_requests - (int32_t)run.size() - (int32_t)waiting.size();
  r->mean_active = step ? active_sum / (double)step : 0.0;
  return KARA_OK;
}

}  // extern "C"
