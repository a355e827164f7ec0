// An in-order queue of jobs served by one host thread.
//
// The layer pipeline hands work that would hold up the thread enqueuing a
// layer's attention to such workers: the copy half of a staging step (with
// the DMA engine it blocks on the plan read-back, the packing and the
// memcpy) and, for layers with few (request, KV head) pairs, the whole
// background chain, whose cross-stream waits cost the enqueuing thread
// microseconds each (OasisKV, paperlayer summary, section 4: the per-layer
// chain runs in the background, the foreground waits only for what its own
// attention needs).  Jobs run in submission order; after the first failure
// the rest are dropped and every waiter returns.  Plain C++ (no HIP), so
// that the same code is built and checked under ThreadSanitizer on a
// machine with no GPU.
#pragma once

#include <condition_variable>
#include <deque>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

namespace oasis {

// Job: a copyable type with int members `layer` and `step`.
template <class Job>
class CopyQueue {
  public:
    // Returns 0 on success; otherwise fills *msg and returns an error code.
    using Runner = std::function<int(const Job &, std::string *msg)>;

    CopyQueue() = default;
    CopyQueue(const CopyQueue &) = delete;
    CopyQueue &operator=(const CopyQueue &) = delete;
    ~CopyQueue() { stop(); }

    // Start the worker for layers [0, n_layers).  on_start runs first on the
    // worker thread (to select its device).
    void start(int n_layers, Runner run, std::function<void()> on_start = {}) {
        done_.assign(n_layers, -1);
        run_ = std::move(run);
        worker_ = std::thread([this, on_start] {
            if (on_start) on_start();
            loop();
        });
    }

    bool started() const { return worker_.joinable(); }

    void push(const Job &j) {
        {
            std::lock_guard<std::mutex> lk(mu_);
            jobs_.push_back(j);
        }
        cv_job_.notify_one();
    }

    // Wait until the job of (layer, step) or a later step of that layer has
    // run, or a job has failed.  Returns the first error code (0 if none).
    int wait_done(int layer, int step) {
        std::unique_lock<std::mutex> lk(mu_);
        if (layer < 0 || layer >= (int)done_.size()) return err_;  // not started, or no such layer
        cv_done_.wait(lk, [&] { return done_[layer] >= step || err_ != 0; });
        return err_;
    }

    // Wait until the queue is empty.  Returns the first error code.
    int drain() {
        std::unique_lock<std::mutex> lk(mu_);
        cv_done_.wait(lk, [&] { return jobs_.empty(); });
        return err_;
    }

    // Record a failure from outside the queue (unless one is recorded):
    // later jobs are dropped and every waiter returns.
    void fail(int code, const std::string &msg) {
        {
            std::lock_guard<std::mutex> lk(mu_);
            if (err_ == 0) {
                err_ = code;
                err_msg_ = msg;
            }
        }
        cv_done_.notify_all();
    }

    // The first error code (0 if none) and its message.
    int error(std::string *msg) {
        std::lock_guard<std::mutex> lk(mu_);
        if (err_ != 0 && msg) *msg = err_msg_;
        return err_;
    }

    // Let the worker finish (or, after an error, drop) what is queued, then
    // join it.
    void stop() {
        if (!worker_.joinable()) return;
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_job_.notify_all();
        worker_.join();
    }

  private:
    void loop() {
        for (;;) {
            Job j;
            int rc;
            {
                std::unique_lock<std::mutex> lk(mu_);
                cv_job_.wait(lk, [&] { return stop_ || !jobs_.empty(); });
                if (jobs_.empty()) return;
                j = jobs_.front();
                rc = err_;  // after a failure, later jobs are not run
            }
            std::string msg;
            if (rc == 0) rc = run_(j, &msg);
            {
                std::lock_guard<std::mutex> lk(mu_);
                jobs_.pop_front();
                if (rc != 0 && err_ == 0) {
                    err_ = rc;
                    err_msg_ = msg;
                }
                if (j.step > done_[j.layer]) done_[j.layer] = j.step;
            }
            cv_done_.notify_all();
        }
    }

    Runner run_;
    std::thread worker_;
    std::mutex mu_;  // everything below
    std::condition_variable cv_job_, cv_done_;
    std::deque<Job> jobs_;
    std::vector<int> done_;  // per layer: the last step whose job has run
    bool stop_ = false;
    int err_ = 0;
    std::string err_msg_;
};

}  // namespace oasis
