// Schedule IR of the persistent decode kernel: a task DAG over per-CU queues, synchronised by
// monotonic counters (or one epoch flag per producer), plus the static validator and a CPU
// simulator.  Host-only C++.
//
// Pages: "AutoMegaKernel" explainer, Method (Layer 0 VM queues of wait -> dispatch -> signal on
// monotonic counters; Layer 2 Schedule IR lowered from the model with a ScheduleConfig) and
// Safety Gate (deadlock-freedom, race-freedom, correctness checks before any launch).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/pmk.h"

namespace pmk {

struct ModelDims {
  int L, H, nq, nkv, hd, F, V, max_seq;
  int wdt, kvdt;  // pmk_dtype
  float eps, theta;
  int grp() const { return nq / nkv; }
  int qkv_rows() const { return (nq + 2 * nkv) * hd; }
  int qdim() const { return nq * hd; }
};

struct Counter {
  int producers;  // signals per step
  int flag_base;  // first flag word of this counter in flags mode
  int phase;      // op of its producers (for diagnostics)
  int layer;
};

struct Schedule {
  ModelDims m;
  int n_queues = 0;
  int attn_splits = 1;
  int combine_parts = 1;  // COMBINE tasks per kv head (each over a range of its q heads)
  int o_copy = 0;         // a COMBINE copies its queue's next O-projection tile to LDS before its wait
  int sync_mode = PMK_SYNC_FLAGS;
  std::vector<pmk_task> tasks;
  std::vector<std::vector<int32_t>> queues;  // task indices per queue, in program order (one step)
  std::vector<Counter> counters;
  int n_flags = 0;
  // counter ids
  int c_lm = -1;
  std::vector<int> c_qkv, c_attn, c_cmb, c_oproj, c_gu, c_down;  // c_attn: [L][nkv]
};

// Longest attention split (positions) one task holds in registers.
int attn_max_chunk(const ModelDims& m);

// Relative streaming speed of each queue per GEMV op (indexed by pmk_op; an empty vector means
// equal speeds): the builder gives each GEMV task a row share proportional to its queue's weight.
struct RowWeights {
  std::vector<double> w[8];
};

// Builder: lowers the model into per-queue task lists (one decode step; the kernel repeats it).
std::string build_schedule(const ModelDims& m, const pmk_schedule_config& sc, int n_queues, Schedule* out,
                           const RowWeights* rw = nullptr);

// Static validator; returns "" when the schedule passes, else "<check>: <detail>".
std::string validate_schedule(const Schedule& s);

// CPU simulator (host threads, randomised interleavings, poisoned buffers).
pmk_status simulate_schedule(const Schedule& s, int steps, uint64_t seed, std::string* report);

uint64_t schedule_hash(const Schedule& s);

// Flattened device tables (task array, queue offsets, queue entries, counter table).
struct DeviceTables {
  std::vector<pmk_task> tasks;
  std::vector<int32_t> qoff;    // n_queues + 1
  std::vector<int32_t> qtasks;  // concatenated queue entries
  std::vector<int32_t> ctr_producers;
  std::vector<int32_t> ctr_flag_base;
};
DeviceTables flatten(const Schedule& s);

}  // namespace pmk

struct pmk_schedule {
  pmk::Schedule s;
};
