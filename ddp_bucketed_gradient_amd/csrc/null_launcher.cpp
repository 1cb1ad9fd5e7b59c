// null_launcher.cpp -- Launcher that enqueues nothing. Linked only into the
// host-only test library so the plan and the readiness state machine can be
// exercised on a machine without a GPU. It moves no data: gradients are left
// untouched, so it is never a substitute for the HIP launcher.
#include <atomic>

#include "core.hpp"

namespace {
// Joins requested by every null launcher of the process (read by the host
// tests through ddpb_hostonly_join_count).
std::atomic<long long> g_joins{0};
}  // namespace

namespace ddpb {
namespace {

class NullLauncher final : public Launcher {
 public:
  int bind(const Plan&, const BindArgs&, std::string*) override { return kOk; }
  int launch(int32_t, int32_t, int64_t, std::string*) override { return kOk; }
  int join(std::string*) override {
    ++g_joins;
    return kOk;
  }
  int accumulate(void* const*, int32_t, bool, std::string*) override { return kOk; }
  int read_stamps(const std::vector<LaunchRecord>& log, std::vector<int64_t>* t0, std::vector<int64_t>* t1,
                  std::string*) override {
    t0->assign(log.size(), 0);
    t1->assign(log.size(), 0);
    return kOk;
  }
  int read_times(int64_t, const std::vector<LaunchRecord>&, std::vector<float>*, std::vector<float>*,
                 std::string* err) override {
    *err = "no device in the host-only test build";
    return kErrState;
  }
  void set_max_blocks(int32_t) override {}
  int set_workgroups_per_cu(int32_t, std::string*) override { return kOk; }
  int set_used(const uint8_t*, const uint8_t*, std::string*) override { return kOk; }
  int set_sync_step(void* const*, int32_t, bool, std::string*) override { return kOk; }
  int clock_hz(int64_t* hz, std::string*) override {
    *hz = 0;
    return kOk;
  }
};

}  // namespace

std::unique_ptr<Launcher> make_launcher() { return std::make_unique<NullLauncher>(); }

}  // namespace ddpb

// Host-only test build: how many times the state machine asked a launcher to
// make the compute stream wait for the side streams.
extern "C" long long ddpb_hostonly_join_count(void) { return g_joins.load(); }
