// Driver for the ThreadSanitizer build of the schedule simulator (host code only, built with g++ by
// tests/test_schedule_validator.py): lowers small models, runs the multi-threaded simulator on
// each, and runs it on a schedule the validator rejects for a race, so that both the clean and the
// failing paths of the simulator run under the sanitizer.  Exit status 0 when every simulation
// ends as expected.
#include <cstdio>
#include <string>

#include "../persistent_megakernel_02_amd/csrc/schedule.h"

int main() {
  int bad = 0;
  for (int n_queues : {2, 5, 8}) {
    for (int mode : {PMK_SYNC_FLAGS, PMK_SYNC_COUNTERS}) {
      pmk::ModelDims m{2, 256, 4, 2, 64, 688, 1024, 48, PMK_DT_F16, PMK_DT_F16, 1e-5f, 10000.f};
      pmk_schedule_config sc{};
      sc.sync_mode = mode;
      pmk::Schedule s;
      std::string e = pmk::build_schedule(m, sc, n_queues, &s);
      if (e.empty()) e = pmk::validate_schedule(s);
      std::string rep;
      const pmk_status st = e.empty() ? pmk::simulate_schedule(s, 3, 7, &rep) : PMK_ERR_SCHEDULE_INVALID;
      std::printf("queues %d mode %d: %s %s\n", n_queues, mode, e.c_str(), rep.c_str());
      bad += st != PMK_OK;
      // the down projections of layer 0 no longer wait for the gate/up tasks whose h they read
      for (auto& t : s.tasks)
        if (t.op == PMK_OP_DOWN && t.layer == 0) t.wait_ctr = -1;
      rep.clear();
      const pmk_status st2 = pmk::simulate_schedule(s, 2, 11, &rep);
      std::printf("  without the down waits: %d %s\n", (int)st2, rep.c_str());
      bad += st2 == PMK_ERR_TIMEOUT;  // a race or a clean run are both possible outcomes; no hang
    }
  }
  return bad ? 1 : 0;
}
