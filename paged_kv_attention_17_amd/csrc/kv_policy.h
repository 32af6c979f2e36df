// The cache policy of the decode calls' K/V reads (pkv_set_kv_read_policy):
// the process-wide setting, and a per-thread override that the library's own
// callers (the scheduler) set around the calls they enqueue.  Host only;
// internal to the library.
#pragma once

namespace pkv {

// PKV_KV_READ_STREAM or PKV_KV_READ_REUSE: this thread's override if set,
// else the process-wide setting.
int kv_read_policy_now();

// Sets this thread's override (0 clears it); returns the previous override.
int kv_read_override(int policy);

// The process-wide setting (pkv_set_kv_read_policy / pkv_kv_read_policy).
void kv_read_set(int policy);
int kv_read_setting();

// Holds an override for the lifetime of the object.
class KvReadScope {
 public:
  explicit KvReadScope(int policy) : prev_(kv_read_override(policy)) {}
  ~KvReadScope() { kv_read_override(prev_); }
  KvReadScope(const KvReadScope&) = delete;
  KvReadScope& operator=(const KvReadScope&) = delete;

 private:
  int prev_;
};

}  // namespace pkv
