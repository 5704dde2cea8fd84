"""Turn a rocprofv3 --kernel-trace --stats CSV into the short markdown summary kept in profiles/.

    python profiles/summarize.py <run>_kernel_stats.csv "<command that produced it>" > profiles/<name>.md
"""
import csv
import sys


def main():
    path, cmd = sys.argv[1], sys.argv[2]
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("# rocprofv3 kernel statistics\n")
    print("Command (run from /tmp with TMPDIR=/tmp on one MI355X):\n")
    print("```\n" + cmd + "\n```\n")
    print("| calls | avg (us) | min (us) | max (us) | total (ms) | % | kernel |")
    print("|---:|---:|---:|---:|---:|---:|---|")
    for r in rows[:25]:
        name = r["Name"].replace("|", "\\|")
        if len(name) > 110:
            name = name[:107] + "..."
        print(f"| {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
              f"{float(r['Percentage']):.2f} | `{name}` |")


if __name__ == "__main__":
    main()
