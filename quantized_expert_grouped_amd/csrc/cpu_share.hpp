// The host's share of a streamed walk ("#1282 prefill: STRATA_PREFILL_CPU_SHARE=auto hands a
// small chunk's least-routed experts to the idle CPU pool", "What it does"): a pool of host
// threads computes the unweighted rows of the experts handed to it, straight from their raw bytes
// in the pinned host arena, while the GPU streams and computes the rest.  Host code only (built by
// the host compiler); no device code and no HIP calls.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace moe {

// One expert's routed rows through gate/up, SwiGLU with q8_1 requantisation, and down, on the
// host.  The activations are quantised to q8_1 here with the layer's arithmetic (the same bytes the
// GPU's quantiser writes), so the block dots are the same integers; the fp32 sums run in another
// order than the GPU's, so the rows agree with the GPU's to fp32 rounding, not bit for bit.
//   wtype: 0 Q8_0 (DS4 activations), 1 Q4_1 (DS4), 2 Q8_0 with D4 activations
//   expert: the raw expert (gate | up | down, blocks along the reduction dimension)
//   x_rows: n_rows pointers to the fp32 input row (H values) of each routed row
//   out: fp32 [n_rows x H], row j the expert's unweighted output for x_rows[j]
struct CpuScratch {
  std::vector<uint8_t> act;   // q8_1 blocks of the rows' inputs
  std::vector<uint8_t> hq;    // q8_1 blocks of h
  std::vector<float> g, u, h;
};
void cpu_expert_rows(int wtype, int H, int F, const uint8_t* expert, const float* const* x_rows,
                     int n_rows, float* out, CpuScratch& scratch);

// Which instruction set the dot products use on this host ("avx512-vnni", "avx2" or "scalar").
const char* cpu_share_isa();

// A persistent pool: start(n, fn) has the pool's threads call fn(job, worker) for job = 0..n-1
// (workers 1..size()-1) and returns at once; wait() takes jobs on the caller's thread too
// (worker 0) and returns when every job is done.  One start/wait pair at a time.
class CpuPool {
 public:
  explicit CpuPool(int n_threads);
  ~CpuPool();
  int size() const { return (int)workers_.size() + 1; }
  void start(int n_jobs, std::function<void(int, int)> fn);
  void wait();

 private:
  void loop(int worker);
  void work(int worker);
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable go_, done_;
  std::function<void(int, int)> fn_;
  std::atomic<int> next_{0};
  int n_jobs_ = 0, busy_ = 0;
  uint64_t generation_ = 0;
  bool stop_ = false;
};

}  // namespace moe
