// Host-side harness of the C ABI in libq8attn (api.hip), for the sanitizer builds.
//
// api.hip is compiled as plain C++ and linked against this file, which supplies
//   * a fake in-process HIP runtime: every stream is a FIFO of operations (copies, event
//     records, event waits, kernel launches) that run later, when a scheduler picks them; a wait
//     may run only once the record it waits for has run, as on the device.  The scheduler runs
//     the streams in a chosen priority order (copies as early as the events allow, or compute
//     first), so a missing event dependency in the streaming loops shows up as a launch that
//     reads the wrong bytes;
//   * stub kernel launchers that enqueue a launch record whose check runs when the scheduler
//     executes it: the chunk launches of the streamed calls compare the bytes of their device
//     slot with the chunk the host buffers (or files) hold for that position.
// No GPU is used.  tests/test_sanitizers.py builds it with -fsanitize=address,undefined and with
// -fsanitize=thread and runs it; it prints ALL OK and exits 0 when every check holds.
#include <hip/hip_runtime_api.h>

#include <fcntl.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include <deque>
#include <functional>
#include <string>
#include <vector>

#include "q8attn.h"
#include "q8attn_internal.h"

// ------------------------------------------------------------------ checks

static int g_failures = 0;
#define CHECK(cond)                                                                              \
    do {                                                                                         \
        if (!(cond)) {                                                                           \
            fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #cond);             \
            ++g_failures;                                                                        \
        }                                                                                        \
    } while (0)

// ------------------------------------------------------------------ fake runtime

enum OpKind { OP_COPY, OP_RECORD, OP_WAIT, OP_LAUNCH };

struct Op {
    OpKind kind;
    int64_t id;
    // copy
    void *dst = nullptr;
    const void *src = nullptr;
    size_t bytes = 0;
    // record: the event; wait: the record id waited for (-1: none)
    ihipEvent_t *event = nullptr;
    int64_t wait_for = -1;
    // launch
    std::function<void()> run;
};

struct ihipStream_t {
    std::deque<Op> q;
    const char *name;
};

struct ihipEvent_t {
    int64_t last_record = -1; // id of the most recent record op enqueued on it
};

static ihipStream_t g_null_stream{{}, "null"};
static std::vector<char> g_done;       // op id -> executed
static int64_t g_next_id = 0;
static std::vector<ihipStream_t *> g_order; // scheduler priority
static int g_live_events = 0;

static ihipStream_t *S(hipStream_t s) { return s ? s : &g_null_stream; }

static int64_t new_id()
{
    g_done.push_back(0);
    return g_next_id++;
}

static bool runnable(const Op &op)
{
    return op.kind != OP_WAIT || op.wait_for < 0 || g_done[op.wait_for];
}

static void execute(Op &op)
{
    if (op.kind == OP_COPY)
        memcpy(op.dst, op.src, op.bytes);
    else if (op.kind == OP_LAUNCH && op.run)
        op.run();
    g_done[op.id] = 1;
}

// Run queued operations until `until` (an op id) has run (-1: until nothing can run).  Streams
// are tried in g_order, then the null stream.
static void schedule(int64_t until = -1)
{
    std::vector<ihipStream_t *> order = g_order;
    order.push_back(&g_null_stream);
    for (;;) {
        if (until >= 0 && g_done[until])
            return;
        bool progressed = false;
        for (ihipStream_t *s : order) {
            if (!s->q.empty() && runnable(s->q.front())) {
                Op op = std::move(s->q.front());
                s->q.pop_front();
                execute(op);
                progressed = true;
                break; // re-start from the highest-priority stream
            }
        }
        if (!progressed)
            break;
    }
    bool pending = false;
    for (ihipStream_t *s : order)
        pending = pending || !s->q.empty();
    if (until >= 0)
        CHECK(g_done[until]); // a host wait that could never end would hang on a device
    else
        CHECK(!pending);      // queued work that can never run (a wait on a later record)
}

static void enqueue(hipStream_t s, Op op)
{
    op.id = new_id();
    S(s)->q.push_back(std::move(op));
}

extern "C" {

hipError_t hipEventCreateWithFlags(hipEvent_t *event, unsigned flags)
{
    (void)flags;
    *event = new ihipEvent_t();
    ++g_live_events;
    return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t event)
{
    delete event;
    --g_live_events;
    return hipSuccess;
}

hipError_t hipEventSynchronize(hipEvent_t event)
{
    if (event->last_record >= 0)
        schedule(event->last_record);
    return hipSuccess;
}

hipError_t hipStreamWaitEvent(hipStream_t stream, hipEvent_t event, unsigned int flags)
{
    (void)flags;
    Op op;
    op.kind = OP_WAIT;
    op.wait_for = event->last_record;
    enqueue(stream, std::move(op));
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t sizeBytes, hipMemcpyKind kind,
                          hipStream_t stream)
{
    (void)kind;
    Op op;
    op.kind = OP_COPY;
    op.dst = dst;
    op.src = src;
    op.bytes = sizeBytes;
    enqueue(stream, std::move(op));
    return hipSuccess;
}

} // extern "C"

// both overloads of hipEventRecord the header declares resolve here
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream)
{
    Op op;
    op.kind = OP_RECORD;
    op.event = event;
    enqueue(stream, std::move(op));
    event->last_record = S(stream)->q.back().id;
    return hipSuccess;
}

// ------------------------------------------------------------------ stub launchers

struct Launch {
    std::string kind;
    q8a::AccumulateArgs a{};
    int kv_dtype = -1;
    int64_t n = 0;
    hipStream_t s = nullptr;
};
static std::vector<Launch> g_log;
static std::function<void(const Launch &)> g_on_run; // per-test check at execution time

static hipError_t record_launch(Launch l)
{
    g_log.push_back(l);
    Op op;
    op.kind = OP_LAUNCH;
    op.run = [l]() {
        if (g_on_run)
            g_on_run(l);
    };
    enqueue(l.s, std::move(op));
    return hipSuccess;
}

namespace q8a {
hipError_t launch_q8_0_pack(const float *, uint8_t *, int64_t n_blocks, hipStream_t s)
{
    Launch l;
    l.kind = "pack";
    l.n = n_blocks;
    l.s = s;
    return record_launch(l);
}
hipError_t launch_q8_0_pack_rows(const float *, const float *, uint8_t *, uint8_t *, int32_t,
                                 int32_t, int32_t n_rows, int64_t, int64_t, hipStream_t s)
{
    Launch l;
    l.kind = "pack_rows";
    l.n = n_rows;
    l.s = s;
    return record_launch(l);
}
hipError_t launch_state_init(float *, float *, int64_t n_rows, hipStream_t s)
{
    Launch l;
    l.kind = "init";
    l.n = n_rows;
    l.s = s;
    return record_launch(l);
}
hipError_t launch_accumulate(const AccumulateArgs &a, int kv_dtype, hipStream_t s)
{
    Launch l;
    l.kind = "accumulate";
    l.a = a;
    l.kv_dtype = kv_dtype;
    l.s = s;
    return record_launch(l);
}
hipError_t launch_finalize(const float *, const float *, const float *, void *, float *,
                           int64_t n_rows, hipStream_t s)
{
    Launch l;
    l.kind = "finalize";
    l.n = n_rows;
    l.s = s;
    return record_launch(l);
}
hipError_t launch_merge(float *, float *, float *, const float *, const float *, const float *,
                        int64_t n_rows, hipStream_t s)
{
    Launch l;
    l.kind = "merge";
    l.n = n_rows;
    l.s = s;
    return record_launch(l);
}
} // namespace q8a

static void reset()
{
    schedule();
    g_log.clear();
    g_on_run = nullptr;
}

static std::string kinds()
{
    std::string r;
    for (auto &l : g_log)
        r += (r.empty() ? "" : ",") + l.kind;
    return r;
}

// ------------------------------------------------------------------ device-like buffers

// 16-byte (or more) aligned host memory standing in for device buffers
struct Buf {
    void *p = nullptr;
    explicit Buf(size_t n, size_t align = 4096)
    {
        p = aligned_alloc(align, (n + align - 1) / align * align);
        memset(p, 0, n);
    }
    ~Buf() { free(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
    template <class T> T *as() const { return static_cast<T *>(p); }
};

static uint8_t pattern(int64_t chunk, int64_t off, int tensor)
{
    return (uint8_t)((chunk * 131 + off * 7 + tensor * 59 + (off >> 8)) & 0xFF);
}

// ------------------------------------------------------------------ tests

static void test_validation()
{
    Buf q(1 << 16), m(1 << 16), l(1 << 16), o(1 << 20), k(1 << 20), v(1 << 20);
    q8a_state st{};
    CHECK(attn_state_init(&st, m.as<float>(), l.as<float>(), o.as<float>(), 1, 4, 256, 128, 0,
                          nullptr) == Q8A_E_UNSUPPORTED);
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>() + 2, 1, 4,
                                   256, 64, 0) == Q8A_E_ALIGN);
    CHECK(st.magic == 0);
    CHECK(g_log.empty());
    CHECK(attn_state_init(&st, m.as<float>(), l.as<float>(), o.as<float>(), 1, 4, 256, 64, 0,
                          nullptr) == Q8A_OK);
    CHECK(kinds() == "init" && st.flags == 0);
    reset();
    CHECK(attn_accumulate_chunk(&st, q.p, k.p, v.p, 7, 0, 64, 256 * 68, 0, 1, nullptr) ==
          Q8A_E_INVAL);
    CHECK(attn_accumulate_chunk(&st, q.p, k.as<uint8_t>() + 4, v.p, 0, 0, 64, 256 * 68, 0, 1,
                                nullptr) == Q8A_E_ALIGN);
    CHECK(attn_accumulate_chunk(&st, q.p, k.p, v.p, 0, 0, 64, 64 * 68 - 16, 0, 1, nullptr) ==
          Q8A_E_INVAL);
    CHECK(attn_accumulate_chunk_final(&st, q.p, k.p, v.p, 0, 0, 64, 256 * 68, 0, 0, o.p,
                                      nullptr, nullptr) == Q8A_E_INVAL);
    st.flags = 0x400; // unknown bit
    CHECK(attn_finalize(&st, q.p, nullptr, nullptr) == Q8A_E_STATE);
    st.flags = 0;
    CHECK(g_log.empty());
    reset();
}

static void test_flags()
{
    Buf q(1 << 16), m(1 << 16), l(1 << 16), o(1 << 20), k(1 << 20), v(1 << 20), out(1 << 20);
    q8a_state st{};
    // deferred: no launch; a chunk every row sees: one accumulate launch, fresh, no init
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>(), 1, 4, 256,
                                   64, 100) == Q8A_OK);
    CHECK(g_log.empty() && st.flags == Q8A_STATE_FRESH);
    st.flags |= Q8A_FORM_NARROW | Q8A_STATE_FINAL_OUT_ONLY;
    CHECK(attn_accumulate_chunk_final(&st, q.p, k.p, v.p, 0, 100, 64, 256 * 68, 0, 1, out.p,
                                      nullptr, nullptr) == Q8A_OK);
    CHECK(kinds() == "accumulate");
    CHECK(g_log[0].a.fresh == 1 && g_log[0].a.form == q8a::kFormNarrow &&
          g_log[0].a.final_out_only == 1);
    CHECK(st.flags == (Q8A_FORM_NARROW | Q8A_STATE_FINAL_OUT_ONLY));
    reset();
    // the next call reads the state
    CHECK(attn_accumulate_chunk(&st, q.p, k.p, v.p, 0, 0, 64, 256 * 68, 0, 1, nullptr) ==
          Q8A_OK);
    CHECK(kinds() == "accumulate" && g_log[0].a.fresh == 0 && g_log[0].a.final_out_only == 0);
    reset();
    // a first chunk after q_pos0: the initialisation comes first
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>(), 1, 4, 256,
                                   64, 100) == Q8A_OK);
    CHECK(attn_accumulate_chunk(&st, q.p, k.p, v.p, 0, 101, 64, 256 * 68, 0, 1, nullptr) ==
          Q8A_OK);
    CHECK(kinds() == "init,accumulate" && g_log[1].a.fresh == 0 && st.flags == 0);
    reset();
    // ... unless the mask is off
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>(), 1, 4, 256,
                                   64, 100) == Q8A_OK);
    CHECK(attn_accumulate_chunk(&st, q.p, k.p, v.p, 0, 5000, 64, 256 * 68, 0, 0, nullptr) ==
          Q8A_OK);
    CHECK(kinds() == "accumulate" && g_log[0].a.fresh == 1);
    reset();
    // finalize and merge of fresh states
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>(), 1, 4, 256,
                                   64, 0) == Q8A_OK);
    CHECK(attn_finalize(&st, out.p, nullptr, nullptr) == Q8A_OK);
    CHECK(kinds() == "init,finalize" && st.flags == 0);
    reset();
    Buf m2(1 << 16), l2(1 << 16), o2(1 << 20);
    q8a_state src{};
    CHECK(attn_state_init_deferred(&src, m2.as<float>(), l2.as<float>(), o2.as<float>(), 1, 4,
                                   256, 64, 0) == Q8A_OK);
    CHECK(attn_state_merge(&st, &src, nullptr) == Q8A_OK);
    CHECK(g_log.empty() && src.flags == Q8A_STATE_FRESH);
    st.flags = Q8A_STATE_FRESH;
    src.flags = 0;
    CHECK(attn_state_merge(&st, &src, nullptr) == Q8A_OK);
    CHECK(kinds() == "init,merge" && st.flags == 0);
    reset();
    // append: the pack, then the accumulate with the fresh handling
    Buf kn(1 << 20), vn(1 << 20);
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>(), 1, 4, 256,
                                   64, 0) == Q8A_OK);
    CHECK(attn_append_chunk(&st, q.p, kn.as<float>(), vn.as<float>(), k.p, v.p, 0, 64, 256 * 68,
                            0, 1, nullptr) == Q8A_OK);
    CHECK(kinds() == "pack_rows,accumulate" && g_log[1].a.fresh == 1 && st.flags == 0);
    reset();
}

// The streamed calls: chunk-major host K/V with a distinct byte pattern per chunk; every chunk
// launch must find its chunk's bytes in its slot when it runs.
struct StreamCase {
    int n_seq, n_heads, n_q, chunk;
    int64_t n_total;
    int64_t q_pos0;
};

static void expect_chunks(const StreamCase &c, int64_t chunk_bytes, int64_t n_expected,
                          std::vector<int64_t> &seen)
{
    g_on_run = [&c, chunk_bytes, &seen](const Launch &l) {
        if (l.kind != "accumulate")
            return;
        const int64_t ci = l.a.kv_pos0 / c.chunk;
        CHECK(l.a.kv_pos0 == ci * c.chunk);
        CHECK(l.a.n_kv == (int32_t)std::min<int64_t>(c.chunk, c.n_total - l.a.kv_pos0));
        CHECK(l.a.fresh == (ci == 0 ? 1 : 0));
        for (int t = 0; t < 2; ++t) {
            const uint8_t *p = t ? l.a.v : l.a.k;
            int64_t bad = 0;
            for (int64_t i = 0; i < chunk_bytes; ++i)
                bad += p[i] != pattern(ci, i, t);
            CHECK(bad == 0);
        }
        seen.push_back(ci);
    };
    (void)n_expected;
}

static void test_stream(const StreamCase &c, bool copy_first)
{
    ihipStream_t cs{{}, "compute"}, ds{{}, "copy"};
    g_order = copy_first ? std::vector<ihipStream_t *>{&ds, &cs}
                         : std::vector<ihipStream_t *>{&cs, &ds};
    const int row = 68;
    const int64_t chunk_bytes = (int64_t)c.n_seq * c.n_heads * c.chunk * row;
    const int64_t n_chunks = (c.n_total + c.chunk - 1) / c.chunk;
    Buf kh(chunk_bytes * n_chunks), vh(chunk_bytes * n_chunks);
    for (int64_t ci = 0; ci < n_chunks; ++ci)
        for (int64_t i = 0; i < chunk_bytes; ++i) {
            kh.as<uint8_t>()[ci * chunk_bytes + i] = pattern(ci, i, 0);
            vh.as<uint8_t>()[ci * chunk_bytes + i] = pattern(ci, i, 1);
        }
    const int64_t rows = (int64_t)c.n_seq * c.n_heads * c.n_q;
    Buf q(rows * 128), m(rows * 4), l(rows * 4), o(rows * 256);
    Buf s0(chunk_bytes), s1(chunk_bytes), s2(chunk_bytes), s3(chunk_bytes);
    void *sk[2] = {s0.p, s1.p}, *sv[2] = {s2.p, s3.p};
    q8a_state st{};
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>(), c.n_seq,
                                   c.n_heads, c.n_q, 64, c.q_pos0) == Q8A_OK);
    std::vector<int64_t> seen;
    expect_chunks(c, chunk_bytes, n_chunks, seen);
    CHECK(attn_accumulate_stream(&st, q.p, kh.p, vh.p, Q8A_KV_Q8_0, c.n_total, c.chunk, sk, sv,
                                 1, &cs, &ds) == Q8A_OK);
    CHECK(!(st.flags & Q8A_STATE_FRESH));
    schedule();
    CHECK((int64_t)seen.size() == n_chunks);
    for (int64_t i = 0; i < (int64_t)seen.size(); ++i)
        CHECK(seen[i] == i);
    CHECK(g_live_events == 0);
    reset();
}

static std::string temp_path(const char *tag)
{
    const char *dir = getenv("TMPDIR");
    return std::string(dir ? dir : "/tmp") + "/q8a_harness_" + tag + "_" +
           std::to_string((long)getpid());
}

static void test_file(const StreamCase &c, int64_t file_offset, int64_t truncate_chunk,
                      bool copy_first)
{
    ihipStream_t cs{{}, "compute"}, ds{{}, "copy"};
    g_order = copy_first ? std::vector<ihipStream_t *>{&ds, &cs}
                         : std::vector<ihipStream_t *>{&cs, &ds};
    const int row = 68;
    const int64_t chunk_bytes = (int64_t)c.n_seq * c.n_heads * c.chunk * row;
    const int64_t n_chunks = (c.n_total + c.chunk - 1) / c.chunk;
    const int64_t n_written = truncate_chunk >= 0 ? truncate_chunk : n_chunks;
    std::string paths[2] = {temp_path("k"), temp_path("v")};
    int fds[2];
    for (int t = 0; t < 2; ++t) {
        fds[t] = open(paths[t].c_str(), O_RDWR | O_CREAT | O_TRUNC, 0600);
        CHECK(fds[t] >= 0);
        std::vector<uint8_t> bytes(file_offset + n_written * chunk_bytes + 100);
        for (size_t i = 0; i < (size_t)file_offset; ++i)
            bytes[i] = 0xEE; // a header before the cache
        for (int64_t ci = 0; ci < n_written; ++ci)
            for (int64_t i = 0; i < chunk_bytes; ++i)
                bytes[file_offset + ci * chunk_bytes + i] = pattern(ci, i, t);
        if (truncate_chunk >= 0) // the file ends inside the first missing chunk
            bytes.resize(file_offset + n_written * chunk_bytes + chunk_bytes / 2);
        CHECK(write(fds[t], bytes.data(), bytes.size()) == (ssize_t)bytes.size());
    }
    const int64_t rows = (int64_t)c.n_seq * c.n_heads * c.n_q;
    Buf q(rows * 128), m(rows * 4), l(rows * 4), o(rows * 256);
    Buf s0(chunk_bytes), s1(chunk_bytes), s2(chunk_bytes), s3(chunk_bytes);
    const int64_t ring_bytes = chunk_bytes + 8192;
    Buf r0(ring_bytes), r1(ring_bytes), r2(ring_bytes), r3(ring_bytes);
    void *sk[2] = {s0.p, s1.p}, *sv[2] = {s2.p, s3.p};
    void *rk[2] = {r0.p, r1.p}, *rv[2] = {r2.p, r3.p};
    q8a_state st{};
    CHECK(attn_state_init_deferred(&st, m.as<float>(), l.as<float>(), o.as<float>(), c.n_seq,
                                   c.n_heads, c.n_q, 64, c.q_pos0) == Q8A_OK);
    std::vector<int64_t> seen;
    expect_chunks(c, chunk_bytes, n_written, seen);
    const int rc = attn_accumulate_file(&st, q.p, fds[0], fds[1], file_offset, Q8A_KV_Q8_0,
                                        c.n_total, c.chunk, rk, rv, ring_bytes, sk, sv, 1, &cs,
                                        &ds);
    CHECK(rc == (truncate_chunk >= 0 ? Q8A_E_IO : Q8A_OK));
    schedule();
    CHECK((int64_t)seen.size() == n_written);
    for (int64_t i = 0; i < (int64_t)seen.size(); ++i)
        CHECK(seen[i] == i);
    CHECK(g_live_events == 0);
    for (int t = 0; t < 2; ++t) {
        close(fds[t]);
        unlink(paths[t].c_str());
    }
    reset();
}

int main()
{
    test_validation();
    test_flags();
    const StreamCase cases[] = {
        {1, 2, 64, 40, 200, 0},     // five full chunks
        {2, 3, 32, 48, 130, 100},   // partial last chunk, two sequences
        {1, 1, 16, 64, 64, 0},      // one chunk
        {1, 2, 16, 32, 70, 0},      // two full chunks and a partial one
    };
    for (const StreamCase &c : cases)
        for (bool copy_first : {true, false}) {
            test_stream(c, copy_first);
            test_file(c, 0, -1, copy_first);
            test_file(c, 1000, -1, copy_first);
            if ((c.n_total + c.chunk - 1) / c.chunk > 1)
                test_file(c, 1000, (c.n_total + c.chunk - 1) / c.chunk - 1, copy_first);
            test_file(c, 4096, 0, copy_first);
        }
    if (g_failures) {
        fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    printf("ALL OK\n");
    return 0;
}
