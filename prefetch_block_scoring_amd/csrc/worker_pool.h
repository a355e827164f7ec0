// A pool of host worker threads that runs one indexed job at a time.
//
// The DMA copy engine packs the admitted blocks of a staging step (OasisKV,
// paperlayer summary, section 4: admitted blocks move host -> HBM in the
// background) on these threads.  Plain C++ (no HIP), so that the same code
// is built and checked under ThreadSanitizer on a machine with no GPU.
#pragma once

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace oasis {

class WorkerPool {
  public:
    WorkerPool() = default;
    WorkerPool(const WorkerPool &) = delete;
    WorkerPool &operator=(const WorkerPool &) = delete;

    ~WorkerPool() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto &t : threads_) t.join();
    }

    // Run fn(i) for every i in [0, n) on up to `want` threads, the caller
    // included, and return when all have finished.  Whatever fn wrote is
    // visible to the caller afterwards.  Calls from several threads are
    // served one after another.
    void run(int want, int n, const std::function<void(int)> &fn) {
        if (n <= 0) return;
        std::lock_guard<std::mutex> run_lk(run_mu_);
        if (want < 1) want = 1;
        ensure(want - 1);
        int helpers;
        {
            std::lock_guard<std::mutex> lk(mu_);
            helpers = std::min<int>(want - 1, (int)threads_.size());
            fn_ = &fn;
            n_ = n;
            next_.store(0);
            active_ = helpers;
            helpers_ = helpers;
            gen_++;
        }
        cv_.notify_all();
        drain(&fn, n);
        std::unique_lock<std::mutex> lk(mu_);
        done_cv_.wait(lk, [&] { return active_ == 0; });
        fn_ = nullptr;
    }

    int threads() {
        std::lock_guard<std::mutex> lk(mu_);
        return (int)threads_.size();
    }

  private:
    void ensure(int k) {
        std::lock_guard<std::mutex> lk(mu_);
        while ((int)threads_.size() < k) {
            const int id = (int)threads_.size();
            threads_.emplace_back([this, id] { loop(id); });
        }
    }

    // take indices until none is left
    void drain(const std::function<void(int)> *fn, int n) {
        for (int i = next_.fetch_add(1); i < n; i = next_.fetch_add(1)) (*fn)(i);
    }

    void loop(int id) {
        uint64_t seen = 0;
        for (;;) {
            const std::function<void(int)> *fn;
            int n;
            {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return stop_ || (gen_ != seen && id < helpers_); });
                if (stop_) return;
                seen = gen_;
                fn = fn_;
                n = n_;
            }
            drain(fn, n);
            {
                std::lock_guard<std::mutex> lk(mu_);
                if (--active_ == 0) done_cv_.notify_all();
            }
        }
    }

    std::mutex run_mu_;  // one job at a time
    std::mutex mu_;      // everything below
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> threads_;
    const std::function<void(int)> *fn_ = nullptr;
    std::atomic<int> next_{0};
    int n_ = 0;
    int active_ = 0;
    int helpers_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

}  // namespace oasis
