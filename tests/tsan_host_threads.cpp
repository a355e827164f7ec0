// Stress of the library's two host-thread components, built with
// ThreadSanitizer by tests/test_host_threads_tsan.py (no GPU needed):
//
//   WorkerPool (worker_pool.h): the DMA engine's packing threads.  Every job
//   writes plain (non-atomic) memory on the helper threads; the caller reads
//   it after run() returns, so a missing happens-before edge is a reported
//   race.  Several callers share one pool, and the helper count changes from
//   job to job.
//
//   CopyQueue (copy_queue.h): the layer pipeline's copy worker.  A producer
//   issues layer-steps in the pipeline's order, waits for step t - 1 of a
//   layer before reading what that job wrote (plain memory again), drains,
//   and in a second round one job fails: later jobs must not run, every
//   waiter must return, and the first error must be the one reported.  Two
//   queues chained as the pipeline's issue threads chain them: a failure in
//   the first releases the producer waiting on the second.
//
// Exit status 0 when every check holds; ThreadSanitizer itself exits with 66
// when it reported anything.
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <thread>
#include <vector>

#include "copy_queue.h"
#include "worker_pool.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            std::exit(1);                                                 \
        }                                                                 \
    } while (0)

static void pool_stress() {
    oasis::WorkerPool pool;
    const int n_callers = 3, jobs = 300;
    std::vector<std::thread> callers;
    std::atomic<long> total{0};
    for (int c = 0; c < n_callers; c++) {
        callers.emplace_back([&, c] {
            std::vector<long> out;
            for (int j = 0; j < jobs; j++) {
                const int n = 1 + (j * 7 + c) % 97;
                const int want = 1 + (j + c) % 16;
                out.assign(n, 0);
                pool.run(want, n, [&](int i) { out[i] = (long)i * i + j; });
                long s = 0;
                for (int i = 0; i < n; i++) {
                    CHECK(out[i] == (long)i * i + j);
                    s += out[i];
                }
                total += s;
            }
        });
    }
    for (auto &t : callers) t.join();
    CHECK(total.load() > 0);
    CHECK(pool.threads() <= 15);
}

struct Job {
    int layer = 0, step = 0;
};

static void queue_round(int layers, int steps, int fail_layer, int fail_step) {
    // written by the worker, read by the producer after wait_done / drain
    std::vector<std::vector<long>> written(layers, std::vector<long>(steps, -1));
    std::vector<int> ran;  // order of the jobs run (worker only, read after drain)
    oasis::CopyQueue<Job> q;
    std::atomic<int> started{0};
    q.start(
        layers,
        [&](const Job &j, std::string *msg) {
            if (j.step % 5 == 0) std::this_thread::sleep_for(std::chrono::microseconds(50));
            if (j.layer == fail_layer && j.step == fail_step) {
                *msg = "job " + std::to_string(j.layer) + "/" + std::to_string(j.step) + " failed";
                return 7;
            }
            written[j.layer][j.step] = 1000L * j.layer + j.step;
            ran.push_back(j.layer * steps + j.step);
            return 0;
        },
        [&] { started++; });
    CHECK(q.started());
    bool failed = false;
    for (int t = 0; t < steps; t++) {
        for (int l = 0; l < layers; l++) {
            if (t >= 1) {
                const int rc = q.wait_done(l, t - 1);
                if (rc != 0) {
                    failed = true;
                } else {
                    CHECK(written[l][t - 1] == 1000L * l + t - 1);
                }
            }
            q.push(Job{l, t});
        }
    }
    const int rc = q.drain();
    std::string msg;
    const int err = q.error(&msg);
    CHECK(rc == err);
    CHECK(started.load() == 1);
    if (fail_layer < 0) {
        CHECK(err == 0 && !failed);
        CHECK((int)ran.size() == layers * steps);
        for (int i = 0; i < (int)ran.size(); i++) {
            // submission order: step-major, layer-minor
            const int t = i / layers, l = i % layers;
            CHECK(ran[i] == l * steps + t);
        }
    } else {
        CHECK(err == 7);
        CHECK(msg == "job " + std::to_string(fail_layer) + "/" + std::to_string(fail_step) + " failed");
        // nothing after the failed job ran
        const int fail_pos = fail_step * layers + fail_layer;
        CHECK((int)ran.size() == fail_pos);
        for (int l = 0; l < layers; l++)
            for (int t = 0; t < steps; t++)
                CHECK((written[l][t] >= 0) == (t * layers + l < fail_pos));
    }
    q.stop();
    q.stop();  // a second stop is a no-op
}

static void queue_stop_with_pending() {
    // stop() lets the worker finish what is queued before it joins
    std::atomic<int> n{0};
    {
        oasis::CopyQueue<Job> q;
        q.start(2, [&](const Job &, std::string *) {
            std::this_thread::sleep_for(std::chrono::microseconds(20));
            n++;
            return 0;
        });
        for (int t = 0; t < 50; t++) q.push(Job{t % 2, t / 2});
    }  // destructor stops
    CHECK(n.load() == 50);
}

// The layer pipeline's issue threads: the producer enqueues each
// layer-step's chain job on one queue, whose runner hands a copy job on to a
// second queue; before the job of (layer, t) the producer waits until the
// copy of (layer, t - 1) has run.  A chain job that fails marks the copy
// queue failed, so that the producer's wait returns.
static void two_queue_handoff(int layers, int steps, int fail_layer, int fail_step) {
    oasis::CopyQueue<Job> copies, chain;
    std::vector<std::vector<long>> issued(layers, std::vector<long>(steps, -1));  // written by the copy worker
    copies.start(layers, [&](const Job &j, std::string *) {
        issued[j.layer][j.step] = 7L * j.layer + j.step;
        return 0;
    });
    chain.start(layers, [&](const Job &j, std::string *msg) {
        if (j.layer == fail_layer && j.step == fail_step) {
            *msg = "chain failed";
            copies.fail(5, *msg);
            return 5;
        }
        copies.push(j);
        return 0;
    });
    bool stopped = false;
    for (int t = 0; t < steps && !stopped; t++) {
        for (int l = 0; l < layers; l++) {
            if (t >= 1) {
                if (copies.wait_done(l, t - 1) != 0) {
                    stopped = true;
                    break;
                }
                CHECK(issued[l][t - 1] == 7L * l + t - 1);
            }
            chain.push(Job{l, t});
        }
    }
    (void)chain.drain();
    (void)copies.drain();
    std::string msg;
    if (fail_layer < 0) {
        CHECK(!stopped && chain.error(&msg) == 0 && copies.error(&msg) == 0);
        for (int l = 0; l < layers; l++)
            for (int t = 0; t < steps; t++) CHECK(issued[l][t] == 7L * l + t);
    } else {
        CHECK(stopped);
        CHECK(chain.error(&msg) == 5 && msg == "chain failed");
        CHECK(copies.error(&msg) == 5);
    }
    chain.stop();
    copies.stop();
}

int main() {
    pool_stress();
    for (int rep = 0; rep < 20; rep++) queue_round(4, 40, -1, -1);
    queue_round(4, 40, 2, 17);
    queue_round(3, 10, 0, 1);
    queue_round(1, 5, 0, 4);
    queue_stop_with_pending();
    for (int rep = 0; rep < 10; rep++) two_queue_handoff(4, 30, -1, -1);
    two_queue_handoff(4, 30, 1, 9);
    two_queue_handoff(2, 5, 0, 0);
    std::printf("host threads: all checks passed\n");
    return 0;
}
