// Schedule builder, static validator and CPU simulator for the persistent decode kernel.
//
// Pages: "AutoMegaKernel" explainer — Method, Layer 2 (the model is lowered into a typed task
// DAG synchronised by monotonic counters, shaped by a ScheduleConfig: tiling, CU allocation,
// pipelining) and the Safety Gate (a schedule is rejected before launch unless the
// producer/consumer DAG is acyclic, every wait threshold t satisfies 1 <= t <= #producers,
// per-queue order is valid, multi-producer counters are joined, memory accesses respect
// happens-before, outputs are reachable and references are intact).  "Kog AI MI300X
// monokernel tutorial": work is split over a fixed grid of CUs ahead of time.
#include "schedule.h"

#include "pmk_limits.h"

#include <algorithm>
#include <cmath>
#include <atomic>
#include <chrono>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <random>
#include <set>
#include <sstream>
#include <thread>

namespace pmk {

namespace {

std::string fmt(const char* f, long a = 0, long b = 0, long c = 0, long d = 0, long e = 0) {
  char buf[512];
  snprintf(buf, sizeof buf, f, a, b, c, d, e);
  return buf;
}

const char* op_name(int op) {
  switch (op) {
    case PMK_OP_QKV: return "QKV";
    case PMK_OP_ATTN: return "ATTN";
    case PMK_OP_OPROJ: return "OPROJ";
    case PMK_OP_GATEUP: return "GATEUP";
    case PMK_OP_DOWN: return "DOWN";
    case PMK_OP_LMHEAD: return "LMHEAD";
    case PMK_OP_TOKEN: return "TOKEN";
    case PMK_OP_COMBINE: return "COMBINE";
  }
  return "?";
}

// Split `n` units into `parts` contiguous ranges; range i = [lo, hi).
void split_range(int n, int parts, int i, int* lo, int* hi) {
  *lo = (int)((int64_t)n * i / parts);
  *hi = (int)((int64_t)n * (i + 1) / parts);
}

}  // namespace

int attn_max_chunk(const ModelDims& m) {
  (void)m;
  return kAttnMaxChunk;
}

// ================================================================================================
// Builder
// ================================================================================================
// Split `units` into `parts` contiguous non-empty ranges with sizes proportional to w[0..parts)
// (cumulative rounding); requires units >= parts.
void split_weighted(int units, int parts, const std::vector<double>& w, std::vector<int>* bounds) {
  double tot = 0;
  for (int i = 0; i < parts; ++i) tot += std::max(w[i], 1e-9);
  bounds->assign(parts + 1, 0);
  double acc = 0;
  for (int i = 0; i < parts; ++i) {
    acc += std::max(w[i], 1e-9);
    (*bounds)[i + 1] = (int)std::llround((double)units * acc / tot);
  }
  for (int i = 1; i < parts; ++i) (*bounds)[i] = std::max((*bounds)[i], (*bounds)[i - 1] + 1);  // non-empty
  (*bounds)[parts] = units;
  for (int i = parts - 1; i > 0; --i) (*bounds)[i] = std::min((*bounds)[i], (*bounds)[i + 1] - 1);
}

std::string build_schedule(const ModelDims& m, const pmk_schedule_config& sc, int n_queues, Schedule* out,
                           const RowWeights* rw) {
  if (n_queues <= 0) return "builder: no queues";
  Schedule s;
  s.m = m;
  s.n_queues = n_queues;
  s.sync_mode = sc.sync_mode == PMK_SYNC_COUNTERS ? PMK_SYNC_COUNTERS : PMK_SYNC_FLAGS;
  int S = sc.attn_splits;
  if (S <= 0) {
    // one split per queue and kv head, but at least two 32-position groups per split: shorter
    // splits leave most of a task's waves idle and multiply the partials the combine reads
    // (2B, 1280 positions: 64 splits of 20 positions 789 tok/s, 20 splits of 64 807)
    S = std::max(1, n_queues / m.nkv);
    S = std::min(S, std::max(1, m.max_seq / 64));
  }
  // each split's positions must fit the attention task (8 waves x 2 x 32): chunk = ceil(max_seq / S)
  // rounded up to whole 32-position blocks is bounded
  const int max_chunk = attn_max_chunk(m);
  S = std::max(S, (m.max_seq + max_chunk - 1) / max_chunk);
  s.attn_splits = S;
  // the combine's early copy of the next O-projection tile: it hides behind the combine's wait when
  // the splits are long (8B class, 4096+ positions in 32 splits: +1 %), and delays the combine's
  // polls when they are short (~1B and 2B, 32 and 64 positions per split: -4 %)
  if (sc.combine_o_copy < 0 || sc.combine_o_copy > 2) return "builder: combine_o_copy must be 0, 1 or 2";
  s.o_copy = sc.combine_o_copy == 2 || (sc.combine_o_copy == 0 && (m.max_seq + S - 1) / S >= 128) ? 1 : 0;
  s.queues.assign(n_queues, {});

  auto add_counter = [&](int producers, int phase, int layer) {
    Counter c{producers, s.n_flags, phase, layer};
    s.n_flags += producers;
    s.counters.push_back(c);
    return (int)s.counters.size() - 1;
  };
  const int L = m.L;
  const int n_qkv = std::min(n_queues, m.qkv_rows() / 2);
  const int n_attn = m.nkv * S;
  // COMBINE of kv head g runs on the queue of its last split (the shortest one), right after it;
  // the O projection then skips those queues when enough others remain, so a combine's latency
  // never delays an O-projection tile.  A combine reads every split's partial of its heads, one
  // batch of loads per thread per 32 splits: when that is more than ~33 KiB for one CU, the
  // head group is split over CP combines (a divisor of the group, each on the queue of one of the
  // last CP splits), as long as the O-projection tiles of the remaining queues still fit the LDS
  // tile area (~128 KiB).
  const int grp = m.grp();
  const int epl = weight_epl(m.wdt);
  const int64_t o_slices = ((int64_t)m.qdim() / epl + 63) / 64;
  const int64_t cbytes = (int64_t)S * grp * (m.hd + 4) * 4;
  // O-projection tile rows (in 1 KiB units) that fit the LDS tile area
  constexpr int64_t kOTileUnits = 136;
  // the largest O tile when the combine queues take no O rows (excl) or half a share each
  auto o_units = [&](int cp, bool half_on_comb) {
    const int64_t nc = (int64_t)m.nkv * cp, no = n_queues - nc;
    const double shares = half_on_comb ? no + 0.5 * nc : (double)no;
    return (int64_t)std::ceil(m.H / shares + 1e-9) * o_slices;
  };
  auto o_fits = [&](int cp) {
    if ((int64_t)m.nkv * cp * 2 > n_queues) return cp == 1;
    return cp == 1 || o_units(cp, false) <= kOTileUnits || o_units(cp, true) <= kOTileUnits;
  };
  int CP = 1;
  if (sc.combine_parts > 0) {
    if (grp % sc.combine_parts) return "builder: combine_parts must divide the q heads per kv head";
    CP = sc.combine_parts;
  } else {
    for (int d = 1; d <= grp; ++d)
      if (grp % d == 0 && o_fits(d)) {
        CP = d;
        if (cbytes / d <= 33 * 1024) break;
      }
  }
  s.combine_parts = CP;
  // with several combines per head group and O tiles that would not fit the queues left, the
  // combine queues keep half an O-projection share each (a short tile, copied by the combine before
  // its wait); the ScheduleConfig can ask for none, half or a full share
  const int share = sc.combine_o_share;
  const bool o_on_comb = share == 2 || share == 3 || (share == 0 && CP > 1 && o_units(CP, false) > kOTileUnits);
  const bool o_half = share != 3;
  auto comb_queue = [&](int g, int p) { return (g * S + S - 1 - p % S + n_queues) % n_queues; };
  std::vector<char> comb_q(n_queues, 0);
  for (int g = 0; g < m.nkv; ++g)
    for (int p = 0; p < CP; ++p) comb_q[comb_queue(g, p)] = 1;
  std::vector<int> o_queues;
  for (int q = 0; q < n_queues; ++q)
    if (!comb_q[q] || o_on_comb) o_queues.push_back(q);
  if ((int)o_queues.size() * 2 < n_queues) {
    o_queues.clear();
    for (int q = 0; q < n_queues; ++q) o_queues.push_back(q);
  }
  const int n_o = std::min((int)o_queues.size(), m.H);
  std::vector<int> o_bounds;  // row bounds of the O tiles when the combine queues take half shares
  if (o_on_comb && o_half && n_o == (int)o_queues.size()) {
    std::vector<double> w(n_o);
    for (int i = 0; i < n_o; ++i) w[i] = comb_q[o_queues[i]] ? 0.5 : 1.0;
    split_weighted(m.H, n_o, w, &o_bounds);
  }
  const int n_gu = std::min(n_queues, m.F);
  const int n_down = std::min(n_queues, m.H);
  const int n_lm = std::min(n_queues, m.V);
  for (int l = 0; l < L; ++l) {
    s.c_qkv.push_back(add_counter(n_qkv, PMK_OP_QKV, l));
    for (int g = 0; g < m.nkv; ++g) s.c_attn.push_back(add_counter(S, PMK_OP_ATTN, l));
    s.c_cmb.push_back(add_counter(m.nkv * CP, PMK_OP_COMBINE, l));
    s.c_oproj.push_back(add_counter(n_o, PMK_OP_OPROJ, l));
    s.c_gu.push_back(add_counter(n_gu, PMK_OP_GATEUP, l));
    s.c_down.push_back(add_counter(n_down, PMK_OP_DOWN, l));
  }
  s.c_lm = add_counter(n_lm, PMK_OP_LMHEAD, -1);

  auto push = [&](int q, pmk_task t) {
    s.tasks.push_back(t);
    s.queues[q].push_back((int32_t)s.tasks.size() - 1);
  };
  // row range of task i of a GEMV op over `units` (rows, or row pairs) split `parts` ways; task i
  // runs on queue qmap[i] (queue i without a map), whose weight sizes its share
  std::vector<int> wb;
  auto split_op = [&](int op, int units, int parts, int i, int* lo, int* hi, const std::vector<int>* qmap = nullptr) {
    if (rw && (int)rw->w[op].size() >= parts) {
      if (i == 0) {
        std::vector<double> w(parts);
        for (int k = 0; k < parts; ++k) w[k] = rw->w[op][qmap ? (*qmap)[k] : k];
        split_weighted(units, parts, w, &wb);
      }
      *lo = wb[i];
      *hi = wb[i + 1];
    } else {
      split_range(units, parts, i, lo, hi);
    }
  };
  for (int l = 0; l < L; ++l) {
    // QKV: packed rows in pairs (each RoPE pair adjacent)
    for (int i = 0; i < n_qkv; ++i) {
      int lo, hi;
      split_op(PMK_OP_QKV, m.qkv_rows() / 2, n_qkv, i, &lo, &hi);
      pmk_task t{PMK_OP_QKV, l, 2 * lo, 2 * hi, -1, 0, 0, s.c_qkv[l], i};
      if (l == 0) { t.wait_ctr = s.c_lm; t.wait_count = n_lm; t.wait_lag = 1; }
      else { t.wait_ctr = s.c_down[l - 1]; t.wait_count = n_down; t.wait_lag = 0; }
      push(i % n_queues, t);
    }
    // ATTN: kv head g, split j, signals the head's counter; COMBINE(g) joins all S splits
    for (int i = 0; i < n_attn; ++i) {
      const int g = i / S, j = i % S;
      push(i % n_queues, pmk_task{PMK_OP_ATTN, l, g, j, s.c_qkv[l], n_qkv, 0, s.c_attn[l * m.nkv + g], j});
    }
    // COMBINE(g, p) merges q heads [j0, j1) of the group, encoded a1 = j0 | j1 << 8
    for (int g = 0; g < m.nkv; ++g)
      for (int p = 0; p < CP; ++p) {
        int j0, j1;
        split_range(grp, CP, p, &j0, &j1);
        push(comb_queue(g, p), pmk_task{PMK_OP_COMBINE, l, g, j0 | (j1 << 8), s.c_attn[l * m.nkv + g], S, 0,
                                        s.c_cmb[l], g * CP + p});
      }
    for (int i = 0; i < n_o; ++i) {
      int lo, hi;
      if (!o_bounds.empty()) {
        lo = o_bounds[i];
        hi = o_bounds[i + 1];
      } else {
        split_op(PMK_OP_OPROJ, m.H, n_o, i, &lo, &hi, &o_queues);
      }
      push(o_queues[i], pmk_task{PMK_OP_OPROJ, l, lo, hi, s.c_cmb[l], m.nkv * CP, 0, s.c_oproj[l], i});
    }
    for (int i = 0; i < n_gu; ++i) {
      int lo, hi;
      split_op(PMK_OP_GATEUP, m.F, n_gu, i, &lo, &hi);
      push(i % n_queues, pmk_task{PMK_OP_GATEUP, l, 2 * lo, 2 * hi, s.c_oproj[l], n_o, 0, s.c_gu[l], i});
    }
    for (int i = 0; i < n_down; ++i) {
      int lo, hi;
      split_op(PMK_OP_DOWN, m.H, n_down, i, &lo, &hi);
      push(i % n_queues, pmk_task{PMK_OP_DOWN, l, lo, hi, s.c_gu[l], n_gu, 0, s.c_down[l], i});
    }
  }
  for (int i = 0; i < n_lm; ++i) {
    int lo, hi;
    split_op(PMK_OP_LMHEAD, m.V, n_lm, i, &lo, &hi);
    push(i % n_queues, pmk_task{PMK_OP_LMHEAD, -1, lo, hi, s.c_down[L - 1], n_down, 0, s.c_lm, i});
  }
  push(0, pmk_task{PMK_OP_TOKEN, -1, 0, 0, s.c_lm, n_lm, 0, -1, 0});
  *out = std::move(s);
  return "";
}

// ================================================================================================
// Access model: what each task reads and writes (shared by the validator and the simulator)
// ================================================================================================
namespace {

enum Buf { B_X = 0, B_XM, B_Q, B_KVCUR, B_PART, B_O, B_H, B_KEY, B_TOKSLOT, B_LOGITS, B_OUT, B_KV, B_COUNT };

// Buffers whose every value carries the step that wrote it: their readers poll the values until the
// tags show the step (in both sync modes), so a tagged read waits for exactly the tasks that write
// the elements it reads.
bool tagged_buf(int b) { return b == B_X || b == B_XM || b == B_Q || b == B_KVCUR || b == B_O; }
enum Kind { A_READ = 0, A_WRITE = 1, A_ATOMIC = 2 };

struct Access {
  int buf;
  int64_t lo, hi;  // element range in the buffer (regions are laid out in one index space per buffer)
  int kind;
  int expect;      // stamp a correct read observes (global step of the write + 1; 0 = initial contents)
};

struct BufDims {
  int64_t size[B_COUNT];
};

BufDims buf_dims(const Schedule& s, int steps) {
  const ModelDims& m = s.m;
  BufDims d;
  d.size[B_X] = (int64_t)(m.L + 1) * m.H;
  d.size[B_XM] = (int64_t)m.L * m.H;
  d.size[B_Q] = (int64_t)m.L * m.qdim();
  d.size[B_KVCUR] = (int64_t)m.L * m.nkv * 2 * m.hd;
  d.size[B_PART] = (int64_t)m.L * m.nkv * s.attn_splits;
  d.size[B_O] = (int64_t)m.L * m.qdim();
  d.size[B_H] = (int64_t)m.L * m.F;
  d.size[B_KEY] = steps + 1;
  d.size[B_TOKSLOT] = 1;
  d.size[B_LOGITS] = (int64_t)(steps + 1) * m.V;
  d.size[B_OUT] = steps + 1;
  d.size[B_KV] = (int64_t)steps * m.L * m.nkv * 2 * m.hd;
  return d;
}

// KV cache: the row each step appends, as (relative step, layer, kv head, K|V, dim); step e writes
// the position pos0 + e, and the attention of a later step reads it from the cache.
int64_t kv_slot(const ModelDims& m, int e, int l, int g, int kv) {
  return ((((int64_t)e * m.L + l) * m.nkv + g) * 2 + kv) * m.hd;
}

// Rows [a0, a1) of the packed QKV matrix -> element ranges written in Q (q heads) and KVCUR (k, v).
// Packed row r in a section is head = r / hd, pair i = (r % hd) / 2, half = r % 2; it holds original
// dimension i + half * hd/2.  A range of whole pairs [p0, p1) of one head covers dims [p0, p1) and
// [p0 + hd/2, p1 + hd/2).
void qkv_writes(const ModelDims& m, int l, int a0, int a1, int e, std::vector<Access>& acc) {
  const int hd = m.hd, half = hd / 2, qrows = m.qdim(), krows = m.nkv * hd;
  for (int r = a0; r < a1;) {
    int sec, base;
    if (r < qrows) { sec = 0; base = 0; }
    else if (r < qrows + krows) { sec = 1; base = qrows; }
    else { sec = 2; base = qrows + krows; }
    const int head = (r - base) / hd;
    const int head_end = base + (head + 1) * hd;
    const int stop = std::min(a1, head_end);
    const int p0 = ((r - base) % hd) / 2, p1 = ((stop - base - 1) % hd) / 2 + 1;
    if (sec == 0) {
      const int64_t off = (int64_t)l * m.qdim() + head * hd;
      acc.push_back({B_Q, off + p0, off + p1, A_WRITE, 0});
      acc.push_back({B_Q, off + half + p0, off + half + p1, A_WRITE, 0});
    } else {
      const int64_t off = ((int64_t)l * m.nkv + head) * 2 * hd + (sec == 2 ? hd : 0);
      acc.push_back({B_KVCUR, off + p0, off + p1, A_WRITE, 0});
      acc.push_back({B_KVCUR, off + half + p0, off + half + p1, A_WRITE, 0});
      // the same dims appended to the cache at this step's position
      const int64_t kv = kv_slot(m, e, l, head, sec - 1);
      acc.push_back({B_KV, kv + p0, kv + p1, A_WRITE, 0});
      acc.push_back({B_KV, kv + half + p0, kv + half + p1, A_WRITE, 0});
    }
    r = stop;
  }
}

// Accesses of task t at global step e (e >= 0).
void task_accesses(const Schedule& s, const pmk_task& t, int e, std::vector<Access>& acc) {
  const ModelDims& m = s.m;
  const int H = m.H, l = t.layer;
  const int W1 = e + 1;  // stamp written at step e
  auto token_read = [&]() {
    if (e == 0) acc.push_back({B_TOKSLOT, 0, 1, A_READ, 0});
    else acc.push_back({B_KEY, e - 1, e, A_READ, e});
  };
  switch (t.op) {
    case PMK_OP_QKV: {
      if (l == 0) token_read();
      else acc.push_back({B_X, (int64_t)l * H, (int64_t)(l + 1) * H, A_READ, W1});
      size_t first = acc.size();
      qkv_writes(m, l, t.a0, t.a1, e, acc);
      for (size_t i = first; i < acc.size(); ++i) acc[i].expect = W1;
      break;
    }
    case PMK_OP_ATTN: {
      const int g = t.a0, grp = m.grp();
      const int64_t part = ((int64_t)l * m.nkv + g) * s.attn_splits;
      acc.push_back({B_Q, (int64_t)l * m.qdim() + (int64_t)g * grp * m.hd,
                     (int64_t)l * m.qdim() + (int64_t)(g + 1) * grp * m.hd, A_READ, W1});
      const int64_t kv = ((int64_t)l * m.nkv + g) * 2 * m.hd;
      acc.push_back({B_KVCUR, kv, kv + 2 * m.hd, A_READ, W1});
      // every row the earlier steps appended (any split may hold a given position)
      for (int e2 = 0; e2 < e; ++e2) acc.push_back({B_KV, kv_slot(m, e2, l, g, 0), kv_slot(m, e2, l, g, 0) + 2 * m.hd, A_READ, e2 + 1});
      acc.push_back({B_PART, part + t.a1, part + t.a1 + 1, A_WRITE, W1});
      break;
    }
    case PMK_OP_COMBINE: {
      const int g = t.a0, grp = m.grp(), j0 = t.a1 & 255, j1 = t.a1 >> 8;
      const int64_t part = ((int64_t)l * m.nkv + g) * s.attn_splits;
      acc.push_back({B_PART, part, part + s.attn_splits, A_READ, W1});
      acc.push_back({B_O, (int64_t)l * m.qdim() + ((int64_t)g * grp + j0) * m.hd,
                     (int64_t)l * m.qdim() + ((int64_t)g * grp + j1) * m.hd, A_WRITE, W1});
      break;
    }
    case PMK_OP_OPROJ:
      acc.push_back({B_O, (int64_t)l * m.qdim(), (int64_t)(l + 1) * m.qdim(), A_READ, W1});
      if (l == 0) token_read();
      else acc.push_back({B_X, (int64_t)l * H + t.a0, (int64_t)l * H + t.a1, A_READ, W1});
      acc.push_back({B_XM, (int64_t)l * H + t.a0, (int64_t)l * H + t.a1, A_WRITE, W1});
      break;
    case PMK_OP_GATEUP:
      acc.push_back({B_XM, (int64_t)l * H, (int64_t)(l + 1) * H, A_READ, W1});
      acc.push_back({B_H, (int64_t)l * m.F + t.a0 / 2, (int64_t)l * m.F + (t.a1 + 1) / 2, A_WRITE, W1});
      break;
    case PMK_OP_DOWN:
      acc.push_back({B_H, (int64_t)l * m.F, (int64_t)(l + 1) * m.F, A_READ, W1});
      acc.push_back({B_XM, (int64_t)l * H + t.a0, (int64_t)l * H + t.a1, A_READ, W1});
      acc.push_back({B_X, (int64_t)(l + 1) * H + t.a0, (int64_t)(l + 1) * H + t.a1, A_WRITE, W1});
      break;
    case PMK_OP_LMHEAD:
      acc.push_back({B_X, (int64_t)m.L * H, (int64_t)(m.L + 1) * H, A_READ, W1});
      acc.push_back({B_LOGITS, (int64_t)e * m.V + t.a0, (int64_t)e * m.V + t.a1, A_WRITE, W1});
      acc.push_back({B_KEY, e, e + 1, A_ATOMIC, W1});
      break;
    case PMK_OP_TOKEN:
      acc.push_back({B_KEY, e, e + 1, A_READ, W1});
      acc.push_back({B_OUT, e, e + 1, A_WRITE, W1});
      acc.push_back({B_TOKSLOT, 0, 1, A_WRITE, W1});
      break;
  }
}

bool valid_op(int op) { return op >= PMK_OP_QKV && op <= PMK_OP_COMBINE; }

// What the kernel executes of a task's declared wait and signal.  In flags mode the consumers of a
// whole step-tagged vector (QKV of layers after the first, ATTN, OPROJ, GATEUP, LMHEAD) poll the
// tags instead of waiting, and the producers of those vectors (QKV, COMBINE, OPROJ, DOWN) publish
// no flag; counters mode executes every declared wait and signal.
int exec_wait(const Schedule& s, const pmk_task& t) {
  if (s.sync_mode == PMK_SYNC_COUNTERS) return t.wait_ctr;
  switch (t.op) {
    case PMK_OP_QKV: return t.layer > 0 ? -1 : t.wait_ctr;
    case PMK_OP_ATTN: case PMK_OP_OPROJ: case PMK_OP_GATEUP: case PMK_OP_LMHEAD: return -1;
    default: return t.wait_ctr;
  }
}
int exec_signal(const Schedule& s, const pmk_task& t) {
  if (s.sync_mode == PMK_SYNC_COUNTERS) return t.signal_ctr;
  switch (t.op) {
    case PMK_OP_QKV: case PMK_OP_COMBINE: case PMK_OP_OPROJ: case PMK_OP_DOWN: return -1;
    default: return t.signal_ctr;
  }
}

// Full-count executed waits are the only counter waits that order a specific producer first.
bool full_wait(const Schedule& s, const pmk_task& t) {
  const int c = exec_wait(s, t);
  return c >= 0 && t.wait_count == s.counters[c].producers;
}

// Is the executed wait of task t at global step e satisfied, given per-(counter, step) counts of
// executed signals?  Counters mode: the counter (the sum over steps) reaches (e - lag) * P + t.
// Flags mode: at least t producers have published step e - lag (producers publish in step order).
bool wait_met(const Schedule& s, const pmk_task& t, int e, const std::vector<int64_t>& sig, int steps) {
  const int c = exec_wait(s, t);
  if (c < 0) return true;
  const int target = e - t.wait_lag;
  if (target < 0) return true;
  if (s.sync_mode == PMK_SYNC_COUNTERS) {
    int64_t total = 0;
    for (int k = 0; k < steps; ++k) total += sig[(size_t)c * steps + k];
    return total >= (int64_t)target * s.counters[c].producers + t.wait_count;
  }
  return sig[(size_t)c * steps + target] >= t.wait_count;
}

// The tasks that write the tagged elements each task reads (the same in every step): tagged reads
// are grouped into lists of writers, one list per distinct (buffer, range) read.
struct TagWaits {
  std::vector<std::vector<int>> lists;     // writers per list
  std::vector<std::vector<int>> of_task;   // lists each task waits on
  std::vector<std::vector<int>> of_writer; // lists each task belongs to
};

TagWaits tag_waits(const Schedule& s) {
  const int NT = (int)s.tasks.size();
  struct W { int64_t lo, hi; int task; };
  std::vector<std::vector<W>> wr(B_COUNT);
  std::vector<Access> acc;
  for (int t = 0; t < NT; ++t) {
    acc.clear();
    task_accesses(s, s.tasks[t], 1, acc);
    for (const Access& a : acc)
      if (tagged_buf(a.buf) && a.kind != A_READ) wr[a.buf].push_back({a.lo, a.hi, t});
  }
  std::vector<std::vector<int64_t>> pmax(B_COUNT);  // prefix max of hi over writes sorted by lo
  for (int b = 0; b < B_COUNT; ++b) {
    std::sort(wr[b].begin(), wr[b].end(), [](const W& x, const W& y) { return x.lo < y.lo; });
    int64_t mx = INT64_MIN;
    for (const W& w : wr[b]) { mx = std::max(mx, w.hi); pmax[b].push_back(mx); }
  }
  TagWaits tw;
  tw.of_task.assign(NT, {});
  tw.of_writer.assign(NT, {});
  std::map<std::tuple<int, int64_t, int64_t>, int> ids;
  for (int t = 0; t < NT; ++t) {
    acc.clear();
    task_accesses(s, s.tasks[t], 1, acc);
    for (const Access& a : acc) {
      if (!tagged_buf(a.buf) || a.kind != A_READ) continue;
      const auto key = std::make_tuple(a.buf, a.lo, a.hi);
      auto it = ids.find(key);
      int id;
      if (it == ids.end()) {
        std::vector<int> ws;
        const auto& v = wr[a.buf];
        // writes with lo < hi of the read, scanned back while some earlier write may still reach lo
        int k = (int)(std::lower_bound(v.begin(), v.end(), a.hi, [](const W& x, int64_t h) { return x.lo < h; }) -
                      v.begin()) - 1;
        for (; k >= 0 && pmax[a.buf][k] > a.lo; --k)
          if (v[k].hi > a.lo) ws.push_back(v[k].task);
        std::sort(ws.begin(), ws.end());
        ws.erase(std::unique(ws.begin(), ws.end()), ws.end());
        id = (int)tw.lists.size();
        tw.lists.push_back(ws);
        for (int w : ws) tw.of_writer[w].push_back(id);
        ids.emplace(key, id);
      } else {
        id = it->second;
      }
      if (std::find(tw.of_task[t].begin(), tw.of_task[t].end(), id) == tw.of_task[t].end()) tw.of_task[t].push_back(id);
    }
  }
  return tw;
}

}  // namespace

// ================================================================================================
// Static validator
// ================================================================================================
std::string validate_schedule(const Schedule& s) {
  const ModelDims& m = s.m;
  const int NT = (int)s.tasks.size(), NQ = s.n_queues, NC = (int)s.counters.size();
  const int S = s.attn_splits;
  // ---- 1. referential integrity ----
  if (NQ <= 0 || (int)s.queues.size() != NQ) return "integrity: queue table size mismatch";
  std::vector<int> seen(NT, 0);
  std::vector<int> queue_of(NT, -1), pos_of(NT, -1);
  for (int q = 0; q < NQ; ++q)
    for (int i = 0; i < (int)s.queues[q].size(); ++i) {
      const int t = s.queues[q][i];
      if (t < 0 || t >= NT) return fmt("integrity: queue %ld entry %ld names task %ld which does not exist", q, i, t);
      if (seen[t]++) return fmt("integrity: task %ld appears in more than one queue slot", t);
      queue_of[t] = q;
      pos_of[t] = i;
    }
  for (int t = 0; t < NT; ++t)
    if (!seen[t]) return fmt("integrity: task %ld is in no queue", t);
  for (int t = 0; t < NT; ++t) {
    const pmk_task& k = s.tasks[t];
    if (!valid_op(k.op)) return fmt("integrity: task %ld has unknown op %ld", t, k.op);
    if (k.wait_ctr < -1 || k.wait_ctr >= NC) return fmt("integrity: task %ld waits on missing counter %ld", t, k.wait_ctr);
    if (k.signal_ctr < -1 || k.signal_ctr >= NC)
      return fmt("integrity: task %ld signals missing counter %ld", t, k.signal_ctr);
    if (k.wait_lag < 0 || k.wait_lag > 1) return fmt("integrity: task %ld has wait lag %ld", t, k.wait_lag);
    const bool layered = k.op != PMK_OP_LMHEAD && k.op != PMK_OP_TOKEN;
    if (layered && (k.layer < 0 || k.layer >= m.L)) return fmt("integrity: task %ld layer %ld out of range", t, k.layer);
    int lim = 0;
    switch (k.op) {
      case PMK_OP_QKV: lim = m.qkv_rows(); break;
      case PMK_OP_OPROJ: case PMK_OP_DOWN: lim = m.H; break;
      case PMK_OP_GATEUP: lim = 2 * m.F; break;
      case PMK_OP_LMHEAD: lim = m.V; break;
      default: break;
    }
    if (k.op == PMK_OP_ATTN) {
      if (k.a0 < 0 || k.a0 >= m.nkv || k.a1 < 0 || k.a1 >= S)
        return fmt("integrity: ATTN task %ld has kv head %ld / split %ld out of range", t, k.a0, k.a1);
    } else if (k.op == PMK_OP_COMBINE) {
      const int j0 = k.a1 & 255, j1 = k.a1 >> 8;
      if (k.a0 < 0 || k.a0 >= m.nkv || k.a1 < 0 || j1 > m.grp() || j0 >= j1)
        return fmt("integrity: COMBINE task %ld has kv head %ld / head range [%ld,%ld) out of range", t, k.a0, j0, j1);
    } else if (lim) {
      if (k.a0 < 0 || k.a1 > lim || k.a0 >= k.a1) return fmt("integrity: task %ld row range [%ld,%ld) invalid", t, k.a0, k.a1);
      if ((k.op == PMK_OP_QKV || k.op == PMK_OP_GATEUP) && ((k.a0 | k.a1) & 1))
        return fmt("integrity: task %ld row range [%ld,%ld) splits a row pair", t, k.a0, k.a1);
      // the GEMV addresses a tile with 32-bit offsets below kMaxTileBytes
      const int64_t K = k.op == PMK_OP_DOWN ? m.F : (k.op == PMK_OP_OPROJ ? m.qdim() : m.H);
      if ((int64_t)(k.a1 - k.a0) * weight_row_bytes(m.wdt, K) > kMaxTileBytes)
        return fmt("integrity: task %ld weight tile of %ld rows exceeds the GEMV's 32-bit offsets", t, k.a1 - k.a0);
    }
  }
  // ---- 2. thresholds and producer counts ----
  std::vector<std::vector<int>> producers(NC);  // tasks that signal c
  for (int t = 0; t < NT; ++t) {
    const pmk_task& k = s.tasks[t];
    if (k.signal_ctr >= 0) producers[k.signal_ctr].push_back(t);
  }
  if (((m.max_seq + S - 1) / S + 31) / 32 * 32 > attn_max_chunk(m))
    return fmt("thresholds: %ld attention splits leave chunks longer than the %ld rows a task holds", S, attn_max_chunk(m));
  std::vector<int> nprod(NC, 0);
  for (int c = 0; c < NC; ++c) nprod[c] = (int)producers[c].size();
  for (int c = 0; c < NC; ++c) {
    if (nprod[c] != s.counters[c].producers)
      return fmt("thresholds: counter %ld declares %ld producers but %ld tasks signal it", c, s.counters[c].producers, nprod[c]);
    std::set<int> slots;
    for (int t : producers[c]) slots.insert(s.tasks[t].signal_slot);
    if ((int)slots.size() != nprod[c] || (nprod[c] && (*slots.begin() != 0 || *slots.rbegin() != nprod[c] - 1)))
      return fmt("thresholds: counter %ld producer slots are not 0..%ld", c, nprod[c] - 1);
  }
  for (int t = 0; t < NT; ++t) {
    const pmk_task& k = s.tasks[t];
    if (k.wait_ctr < 0) continue;
    const int P = s.counters[k.wait_ctr].producers;
    if (k.wait_count < 1 || k.wait_count > P)
      return fmt("thresholds: task %ld waits for %ld signals of counter %ld which has %ld producers", t, k.wait_count, k.wait_ctr, P);
  }
  // ---- 3. deadlock freedom: monotone execution of two steps ----
  // A task runs once its executed counter (or flag) wait is met and every task that writes the
  // step-tagged elements it reads has run in the same step; monotone waits make any fair
  // interleaving reach the same end state, so one greedy pass decides.
  const int STEPS = 2;
  const TagWaits tw = tag_waits(s);
  const int NL = (int)tw.lists.size();
  const int W = NQ;  // vector clock width
  std::vector<int16_t> vc_task((size_t)STEPS * NT * W, -1);
  std::vector<int16_t> join_ctr((size_t)STEPS * NC * W, -1);
  std::vector<int16_t> join_list((size_t)STEPS * NL * W, -1);
  auto vt = [&](int t, int e) { return &vc_task[((size_t)e * NT + t) * W]; };
  auto jc = [&](int c, int e) { return &join_ctr[((size_t)e * NC + c) * W]; };
  auto jl = [&](int k, int e) { return &join_list[((size_t)e * NL + k) * W]; };
  auto vmax = [&](int16_t* a, const int16_t* b) { for (int i = 0; i < W; ++i) a[i] = std::max(a[i], b[i]); };
  {
    std::vector<int64_t> sig((size_t)NC * STEPS, 0);       // executed signals per (counter, step)
    std::vector<int> left((size_t)NL * STEPS, 0);          // writers of each tag list not yet run, per step
    for (int k = 0; k < NL; ++k)
      for (int e = 0; e < STEPS; ++e) left[(size_t)k * STEPS + e] = (int)tw.lists[k].size();
    std::vector<int> head(NQ, 0);  // position in the unrolled queue (step * len + i)
    bool progress = true;
    while (progress) {
      progress = false;
      for (int q = 0; q < NQ; ++q) {
        const int len = (int)s.queues[q].size();
        while (head[q] < STEPS * len) {
          const int e = head[q] / len, t = s.queues[q][head[q] % len];
          const pmk_task& k = s.tasks[t];
          if (!wait_met(s, k, e, sig, STEPS)) break;
          bool tags = true;
          for (int id : tw.of_task[t]) tags = tags && left[(size_t)id * STEPS + e] == 0;
          if (!tags) break;
          // vector clock: program order, the executed full wait's producers, the tag writers
          int16_t* v = vt(t, e);
          if (head[q] > 0) {
            const int pt = s.queues[q][(head[q] - 1) % len], pe = (head[q] - 1) / len;
            std::memcpy(v, vt(pt, pe), W * sizeof(int16_t));
          }
          v[q] = (int16_t)head[q];
          if (full_wait(s, k) && e - k.wait_lag >= 0) vmax(v, jc(exec_wait(s, k), e - k.wait_lag));
          for (int id : tw.of_task[t]) vmax(v, jl(id, e));
          const int c = exec_signal(s, k);
          if (c >= 0) {
            vmax(jc(c, e), v);
            sig[(size_t)c * STEPS + e] += 1;
          }
          for (int id : tw.of_writer[t]) {
            vmax(jl(id, e), v);
            left[(size_t)id * STEPS + e] -= 1;
          }
          ++head[q];
          progress = true;
        }
      }
    }
    for (int q = 0; q < NQ; ++q) {
      const int len = (int)s.queues[q].size();
      if (head[q] < STEPS * len) {
        const int t = s.queues[q][head[q] % len];
        const pmk_task& k = s.tasks[t];
        const int e = head[q] / len;
        std::ostringstream os;
        os << "deadlock: queue " << q << " stalls at step " << e << " on task " << t << " (" << op_name(k.op);
        if (!wait_met(s, k, e, sig, STEPS))
          os << " waits on counter " << exec_wait(s, k) << " for " << k.wait_count << " signals, lag " << k.wait_lag
             << (s.sync_mode == PMK_SYNC_COUNTERS ? "" : ", flags") << ")";
        else
          os << " polls step-tagged data that a task which has not run writes)";
        return os.str();
      }
    }
  }
  // ---- 4/5. happens-before over the two unrolled steps (the vector clocks above) ----
  // node identity for hb queries
  struct Node { int queue, index; const int16_t* vc; };
  auto task_node = [&](int t, int e) { return Node{queue_of[t], e * (int)s.queues[queue_of[t]].size() + pos_of[t], vt(t, e)}; };
  auto hb = [&](const Node& a, const Node& b) { return b.vc[a.queue] >= a.index; };

  // ---- 4. join completeness: a reader of a region written by a multi-producer phase waits on all of it ----
  struct Acc { Access a; Node n; int task; int e; };
  std::vector<std::vector<Acc>> by_buf(B_COUNT);
  std::vector<Access> tmp;
  for (int e = 0; e < STEPS; ++e)
    for (int t = 0; t < NT; ++t) {
      tmp.clear();
      task_accesses(s, s.tasks[t], e, tmp);
      for (auto& a : tmp) by_buf[a.buf].push_back({a, task_node(t, e), t, e});
    }
  for (int t = 0; t < NT; ++t) {
    const pmk_task& k = s.tasks[t];
    if (exec_wait(s, k) < 0 || full_wait(s, k)) continue;
    // executed partial wait: does this task read anything that producers of the waited counter write?
    tmp.clear();
    task_accesses(s, k, 1, tmp);
    std::vector<Access> prod;
    for (int p = 0; p < NT; ++p) {
      const pmk_task& pk = s.tasks[p];
      if (pk.signal_ctr != k.wait_ctr) continue;
      task_accesses(s, pk, 1 - k.wait_lag, prod);
    }
    for (auto& r : tmp)
      if (r.kind == A_READ && !tagged_buf(r.buf))  // a tagged read waits for its own writers
        for (auto& w : prod)
          if (w.kind != A_READ && w.buf == r.buf && w.lo < r.hi && r.lo < w.hi)
            return fmt("join: task %ld reads a region that %ld producers of counter %ld write but waits for only %ld of them",
                       t, s.counters[k.wait_ctr].producers, k.wait_ctr, k.wait_count);
  }
  // ---- 4b. coverage: every element a task reads as a value of some step is written in that step ----
  for (int b = 0; b < B_COUNT; ++b) {
    // merged write intervals per stamp (stamp = step of the write + 1)
    std::map<int, std::vector<std::pair<int64_t, int64_t>>> wr;
    for (const Acc& x : by_buf[b])
      if (x.a.kind != A_READ) wr[x.a.expect].push_back({x.a.lo, x.a.hi});
    for (auto& kv : wr) {
      auto& v = kv.second;
      std::sort(v.begin(), v.end());
      std::vector<std::pair<int64_t, int64_t>> merged;
      for (auto& iv : v) {
        if (!merged.empty() && iv.first <= merged.back().second) merged.back().second = std::max(merged.back().second, iv.second);
        else merged.push_back(iv);
      }
      v.swap(merged);
    }
    for (const Acc& x : by_buf[b]) {
      if (x.a.kind != A_READ || x.a.expect < 1) continue;  // stamp 0: contents from before the first step
      const auto it = wr.find(x.a.expect);
      bool ok = false;
      if (it != wr.end()) {
        const auto& v = it->second;
        auto p = std::upper_bound(v.begin(), v.end(), std::make_pair(x.a.lo, INT64_MAX));
        if (p != v.begin()) {
          --p;
          ok = p->first <= x.a.lo && x.a.hi <= p->second;
        }
      }
      if (!ok) {
        std::ostringstream os;
        os << "coverage: " << op_name(s.tasks[x.task].op) << " task " << x.task << " (step " << x.e << ") reads buffer " << b
           << " elements [" << x.a.lo << ", " << x.a.hi << ") that no task of step " << x.a.expect - 1 << " writes whole";
        return os.str();
      }
    }
  }
  // ---- 5. happens-before on every conflicting pair (within a step and across consecutive steps) ----
  for (int b = 0; b < B_COUNT; ++b) {
    auto& v = by_buf[b];
    std::sort(v.begin(), v.end(), [](const Acc& x, const Acc& y) { return x.a.lo < y.a.lo; });
    for (size_t i = 0; i < v.size(); ++i)
      for (size_t j = i + 1; j < v.size() && v[j].a.lo < v[i].a.hi; ++j) {
        const Acc& x = v[i];
        const Acc& y = v[j];
        if (x.a.kind == A_READ && y.a.kind == A_READ) continue;
        if (x.a.kind == A_ATOMIC && y.a.kind == A_ATOMIC) continue;
        if (x.n.queue == y.n.queue && x.n.index == y.n.index) continue;  // same node
        const Acc* first = &x;
        const Acc* second = &y;
        if (x.e != y.e) {
          if (x.e > y.e) std::swap(first, second);  // across steps: the earlier step's access first
        } else if (x.a.kind == A_READ || y.a.kind == A_READ) {
          // one step, a read and a write: a read of this step's value follows the write; a read of
          // the value from before the step (a lagged read) precedes it
          const Acc* r = x.a.kind == A_READ ? &x : &y;
          const Acc* w = x.a.kind == A_READ ? &y : &x;
          const bool same_step_value = r->a.expect == r->e + 1;
          first = same_step_value ? w : r;
          second = same_step_value ? r : w;
        } else {
          // two writers (or a writer and an atomic) of one step: either order, but ordered
          if (hb(x.n, y.n) || hb(y.n, x.n)) continue;
          return fmt("race: tasks %ld and %ld both write buffer %ld [%ld, ...) in one step without ordering", x.task, y.task, b,
                     (long)std::max(x.a.lo, y.a.lo));
        }
        if (!hb(first->n, second->n)) {
          std::ostringstream os;
          os << "race: " << op_name(s.tasks[first->task].op) << " task " << first->task
             << " (step " << first->e << ", " << (first->a.kind == A_READ ? "read" : "write") << ") is not ordered before "
             << op_name(s.tasks[second->task].op) << " task " << second->task
             << " (step " << second->e << ", " << (second->a.kind == A_READ ? "read" : "write") << ") on buffer " << b
             << " elements [" << std::max(x.a.lo, y.a.lo) << ", " << std::min(x.a.hi, y.a.hi) << ")";
          return os.str();
        }
      }
  }
  // monotonic counters: every executed signal of step e+1 follows every one of step e on a counter
  for (int c = 0; c < NC; ++c) {
    for (int t1 : producers[c]) {
      if (exec_signal(s, s.tasks[t1]) < 0) continue;
      const Node n1 = task_node(t1, 1);
      for (int t0 : producers[c])
        if (!hb(task_node(t0, 0), n1))
          return fmt("counter: task %ld signals counter %ld for step 1 before task %ld has signalled it for step 0", t1, c, t0);
    }
  }
  // ---- 6. output reachability ----
  int tok = -1;
  for (int t = 0; t < NT; ++t)
    if (s.tasks[t].op == PMK_OP_TOKEN) { if (tok >= 0) return "reachability: more than one TOKEN task"; tok = t; }
  if (tok < 0) return "reachability: no TOKEN task (the greedy choice is never read)";
  const Node tn = task_node(tok, 0);
  for (int t = 0; t < NT; ++t)
    if (t != tok && !hb(task_node(t, 0), tn))
      return fmt("reachability: task %ld does not reach the greedy choice of its step (", t) + op_name(s.tasks[t].op) + ")";
  return "";
}

// ================================================================================================
// CPU simulator: one host thread per queue, poisoned stamp buffers, random yields
// ================================================================================================
pmk_status simulate_schedule(const Schedule& s, int steps, uint64_t seed, std::string* report) {
  const int NQ = s.n_queues, NC = (int)s.counters.size();
  BufDims bd = buf_dims(s, steps);
  int64_t total = 0;
  for (int b = 0; b < B_COUNT; ++b) total += bd.size[b];
  if (total > 50'000'000) { *report = "simulate: model too large for the simulator"; return PMK_ERR_INVALID_ARG; }
  std::vector<std::unique_ptr<std::atomic<int32_t>[]>> stamps(B_COUNT);
  for (int b = 0; b < B_COUNT; ++b) {
    stamps[b].reset(new std::atomic<int32_t>[bd.size[b]]);
    for (int64_t i = 0; i < bd.size[b]; ++i) stamps[b][i].store(b == B_TOKSLOT ? 0 : -1);  // -1 = poison
  }
  // executed signals per (counter, step): counters mode sums them, flags mode counts one step's
  std::unique_ptr<std::atomic<int64_t>[]> sig(new std::atomic<int64_t>[(size_t)NC * steps]);
  for (size_t c = 0; c < (size_t)NC * steps; ++c) sig[c].store(0);
  std::atomic<bool> abort_flag{false};
  std::mutex mu;
  std::string first_error;
  pmk_status status = PMK_OK;
  auto fail = [&](pmk_status st, const std::string& msg) {
    std::lock_guard<std::mutex> g(mu);
    if (status == PMK_OK) { status = st; first_error = msg; }
    abort_flag.store(true);
  };
  auto met = [&](const pmk_task& k, int e) {
    const int c = exec_wait(s, k);
    if (c < 0) return true;
    const int target = e - k.wait_lag;
    if (target < 0) return true;
    if (s.sync_mode == PMK_SYNC_COUNTERS) {
      int64_t tot = 0;
      for (int x = 0; x < steps; ++x) tot += sig[(size_t)c * steps + x].load();
      return tot >= (int64_t)target * s.counters[c].producers + k.wait_count;
    }
    return sig[(size_t)c * steps + target].load() >= k.wait_count;
  };
  const auto t_start = std::chrono::steady_clock::now();
  auto stuck = [&](const std::chrono::steady_clock::time_point& t0) {
    return std::chrono::steady_clock::now() - t0 > std::chrono::seconds(5);
  };
  // reads of tagged buffers poll until the element shows this step's stamp (a later step's stamp
  // means it was overwritten before this read: a race); other reads must see it at once
  auto run_accesses = [&](std::mt19937_64& rng, const std::vector<Access>& acc, int e, int phase, const char* what,
                          int task) {
    for (const Access& a : acc) {
      if (a.kind == A_READ && phase != 1) {
        for (int64_t i = a.lo; i < a.hi; ++i) {
          int32_t st = stamps[a.buf][i].load();
          if (phase == 0 && tagged_buf(a.buf) && st < a.expect) {
            const auto t0 = std::chrono::steady_clock::now();
            while ((st = stamps[a.buf][i].load()) < a.expect) {
              if (abort_flag.load()) return;
              std::this_thread::yield();
              if (stuck(t0)) {
                std::ostringstream os;
                os << "deadlock: " << what << " task " << task << " at step " << e << " polled buffer " << a.buf << "[" << i
                   << "] for 5 s (stamp " << st << ", expected " << a.expect << ")";
                fail(PMK_ERR_TIMEOUT, os.str());
                return;
              }
            }
          }
          if (st != a.expect) {
            std::ostringstream os;
            os << "race: " << what << " task " << task << " at step " << e << " read buffer " << a.buf << "[" << i
               << "] with stamp " << st << ", expected " << a.expect << (st < 0 ? " (poisoned)" : "");
            fail(PMK_ERR_SCHEDULE_INVALID, os.str());
            return;
          }
          if ((rng() & 63) == 0) std::this_thread::yield();
        }
      } else if (a.kind != A_READ && phase == 1) {
        for (int64_t i = a.lo; i < a.hi; ++i) {
          stamps[a.buf][i].store(a.expect);
          if ((rng() & 63) == 0) std::this_thread::yield();
        }
      }
    }
  };
  auto worker = [&](int q) {
    std::mt19937_64 rng(seed * 1000003ull + q);
    std::vector<Access> acc;
    const auto& queue = s.queues[q];
    for (int e = 0; e < steps && !abort_flag.load(); ++e) {
      for (int t : queue) {
        const pmk_task& k = s.tasks[t];
        const auto t0 = std::chrono::steady_clock::now();
        while (!met(k, e)) {
          if (abort_flag.load()) return;
          std::this_thread::yield();
          if (stuck(t0)) {
            std::ostringstream os;
            os << "deadlock: queue " << q << " waited 5 s at step " << e << " on counter " << exec_wait(s, k) << " ("
               << op_name(k.op) << " task " << t << ")";
            fail(PMK_ERR_TIMEOUT, os.str());
            return;
          }
        }
        acc.clear();
        task_accesses(s, k, e, acc);
        run_accesses(rng, acc, e, 0, op_name(k.op), t);  // reads at start (tagged ones poll)
        if ((rng() & 3) == 0) std::this_thread::yield();
        run_accesses(rng, acc, e, 1, op_name(k.op), t);  // writes
        run_accesses(rng, acc, e, 2, op_name(k.op), t);  // reads again: catches WAR
        if (abort_flag.load()) return;
        const int c = exec_signal(s, k);
        if (c >= 0) sig[(size_t)c * steps + e].fetch_add(1);
      }
    }
  };
  std::vector<std::thread> th;
  for (int q = 0; q < NQ; ++q) th.emplace_back(worker, q);
  for (auto& t : th) t.join();
  (void)t_start;
  *report = first_error;
  return status;
}

// ================================================================================================
// hashing and flattening
// ================================================================================================
uint64_t schedule_hash(const Schedule& s) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](const void* p, size_t n) {
    const uint8_t* b = (const uint8_t*)p;
    for (size_t i = 0; i < n; ++i) { h ^= b[i]; h *= 1099511628211ull; }
  };
  mix(&s.m, sizeof(s.m));
  mix(&s.n_queues, sizeof(int));
  mix(&s.attn_splits, sizeof(int));
  mix(&s.sync_mode, sizeof(int));
  mix(&s.o_copy, sizeof(int));
  for (auto& t : s.tasks) mix(&t, sizeof(t));
  for (auto& q : s.queues) {
    int n = (int)q.size();
    mix(&n, sizeof n);
    mix(q.data(), q.size() * sizeof(int32_t));
  }
  for (auto& c : s.counters) mix(&c, sizeof c);
  return h;
}

DeviceTables flatten(const Schedule& s) {
  DeviceTables d;
  d.tasks = s.tasks;
  d.qoff.push_back(0);
  for (auto& q : s.queues) {
    d.qtasks.insert(d.qtasks.end(), q.begin(), q.end());
    d.qoff.push_back((int32_t)d.qtasks.size());
  }
  for (auto& c : s.counters) {
    d.ctr_producers.push_back(c.producers);
    d.ctr_flag_base.push_back(c.flag_base);
  }
  return d;
}

}  // namespace pmk
